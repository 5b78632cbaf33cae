// token_cat_quant.hip -- concatenation of the attention and MLP branch rows
// [a | b] fused with static FP8 E4M3 or 16-element-group FP4 (E2M1 values,
// one E4M3 scale per group) quantisation. The bf16 concatenation is never
// written.
//
// What is computed follows the sglang PR 37162 page (the _token_cat_fp8_kernel
// excerpt under "Key source snippets": a column left of the attention width
// reads the attention branch, else the MLP branch; values * (1/scale) clamped
// to the E4M3 range) and the sglang PR 37141 page ("Implementation breakdown"
// item 1: one 16-element group per thread, packed E2M1 codes plus one E4M3
// scale per group, zero scales for pad rows, an inverse global scale).
//
// FP4 group arithmetic (the page leaves it to a third-party primitive; these
// are plain IEEE fp32 steps): s8 = e4m3(min((amax / 6) * g, 448)),
// k = g / value(s8), code = e2m1(x * k); a zero scale gives zero codes.
//
// Layout on gfx950: one wave64 per row. FP8: lane l handles 16-element chunks
// l, l + 64, ... (two 16-byte loads -> one 16-byte store). FP4: lane l handles
// groups l, l + 64, ... (two 16-byte loads -> 8 packed bytes + 1 scale byte;
// the 64 scale bytes of a wave step are contiguous). Chunks and groups never
// straddle the branch boundary because both widths are multiples of 16.
#include "dit_device.h"
#include "kernels.h"

namespace dit {
namespace {

constexpr int kUnroll = 4;

__device__ __forceinline__ const uint16_t* cat_source(const TokenCatArgs& a, int64_t row, int c16) {
    const int a_chunks = (int)(a.a_cols >> 4);
    return c16 < a_chunks ? a.a + row * a.a_cols + 16 * c16
                          : a.b + row * a.b_cols + 16 * (c16 - a_chunks);
}

__global__ __launch_bounds__(256) void token_cat_fp8_kernel(TokenCatArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= a.rows) return;
    const int64_t cols = a.a_cols + a.b_cols;
    const int cpr = (int)(cols >> 4);
    const float inv = 1.0f / *a.scale;  // IEEE division
    uint8_t* orow = a.out + row * cols;

    for (int c0 = 0; c0 < cpr; c0 += 64 * kUnroll) {
        u32x4 lo[kUnroll], hi[kUnroll];
#pragma unroll
        for (int k = 0; k < kUnroll; ++k) {
            const int c = c0 + lane + 64 * k;
            if (c < cpr) {
                const uint16_t* src = cat_source(a, row, c);
                lo[k] = load16(src);
                hi[k] = load16(src + 8);
            }
        }
#pragma unroll
        for (int k = 0; k < kUnroll; ++k) {
            const int c = c0 + lane + 64 * k;
            if (c >= cpr) continue;
            float f[16];
            unpack8(lo[k], *reinterpret_cast<float(*)[8]>(&f[0]));
            unpack8(hi[k], *reinterpret_cast<float(*)[8]>(&f[8]));
            uint32_t w[4];
#pragma unroll
            for (int q = 0; q < 4; ++q)
                w[q] = pack_e4m3x4(clamp_e4m3(f[4 * q] * inv), clamp_e4m3(f[4 * q + 1] * inv),
                                   clamp_e4m3(f[4 * q + 2] * inv), clamp_e4m3(f[4 * q + 3] * inv));
            store16(orow + 16 * c, (u32x4){w[0], w[1], w[2], w[3]});
        }
    }
}

__global__ __launch_bounds__(256) void token_cat_fp4_kernel(TokenCatArgs a, int64_t rows_padded) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows_padded) return;
    const int64_t cols = a.a_cols + a.b_cols;
    const int groups = (int)(cols >> 4);
    uint8_t* srow = a.out_scales + row * groups;
    if (row >= a.rows) {  // pad rows of the scale matrix
        for (int g = lane; g < groups; g += 64) srow[g] = 0;
        return;
    }
    const float gscale = *a.scale;  // global inverse scale
    uint8_t* prow = a.out + row * (cols >> 1);

    for (int g0 = 0; g0 < groups; g0 += 64 * kUnroll) {
        u32x4 lo[kUnroll], hi[kUnroll];
#pragma unroll
        for (int k = 0; k < kUnroll; ++k) {
            const int g = g0 + lane + 64 * k;
            if (g < groups) {
                const uint16_t* src = cat_source(a, row, g);
                lo[k] = load16(src);
                hi[k] = load16(src + 8);
            }
        }
#pragma unroll
        for (int k = 0; k < kUnroll; ++k) {
            const int g = g0 + lane + 64 * k;
            if (g >= groups) continue;
            float f[16];
            unpack8(lo[k], *reinterpret_cast<float(*)[8]>(&f[0]));
            unpack8(hi[k], *reinterpret_cast<float(*)[8]>(&f[8]));
            float amax = 0.0f;
#pragma unroll
            for (int e = 0; e < 16; ++e) amax = __builtin_fmaxf(amax, __builtin_fabsf(f[e]));
            const float s_pre = (amax / 6.0f) * gscale;
            const uint32_t s8 =
                (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(__builtin_fminf(s_pre, 448.0f), 0.0f, 0, false) & 0xFFu;
            u32x2 packed = {0u, 0u};
            if (s8 != 0) {
                const float kq = gscale / e4m3_value_pos(s8);  // IEEE division
                float t0[8], t1[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    t0[e] = f[e] * kq;
                    t1[e] = f[8 + e] * kq;
                }
                packed = (u32x2){pack_e2m1x8(t0), pack_e2m1x8(t1)};
            }
            store8(prow + 8 * g, packed);
            srow[g] = (uint8_t)s8;
        }
    }
}

}  // namespace

hipError_t launch_token_cat_fp8(const TokenCatArgs& a, hipStream_t stream) {
    const dim3 grid((unsigned)((a.rows + 3) / 4));
    hipLaunchKernelGGL(token_cat_fp8_kernel, grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_token_cat_fp4(const TokenCatArgs& a, hipStream_t stream) {
    const int64_t rows_padded = (a.rows + 127) / 128 * 128;
    const dim3 grid((unsigned)((rows_padded + 3) / 4));
    hipLaunchKernelGGL(token_cat_fp4_kernel, grid, dim3(256), 0, stream, a, rows_padded);
    return hipGetLastError();
}

}  // namespace dit

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
// Layout on gfx950: a 2-D grid of (row, tile of chunks). FP8: each lane takes
// 8-element chunks (one 16-byte streaming load -> one 8-byte store), so every
// load instruction of a wave reads 1 KiB contiguously. FP4: one lane per
// 16-element group (two 16-byte loads -> 8 packed bytes + 1 scale byte; a
// wave's 64 scale bytes are contiguous). Chunks and groups never straddle the
// branch boundary because both widths are multiples of 16.
#include "dit_device.h"
#include "kernels.h"

namespace dit {
namespace {

constexpr int kTile = 256;  // chunks (or groups) per workgroup

__device__ __forceinline__ const uint16_t* cat_source(const TokenCatArgs& a, int64_t row, int c16) {
    const int a_chunks = (int)(a.a_cols >> 4);
    return c16 < a_chunks ? a.a + row * a.a_cols + 16 * c16
                          : a.b + row * a.b_cols + 16 * (c16 - a_chunks);
}

__device__ __forceinline__ void load16x2(const uint16_t* src, float (&f)[16]) {
    float lo[8], hi[8];
    unpack8(stream_load16(src), lo);
    unpack8(stream_load16(src + 8), hi);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        f[e] = lo[e];
        f[8 + e] = hi[e];
    }
}

// U chunks per thread, kTile apart: a workgroup covers U * kTile chunks.
// kElems = 16: a chunk is 16 elements (two 16-byte loads, one 16-byte store);
// kElems = 8: a chunk is 8 elements (one 16-byte load, one 8-byte store), so
// each load instruction of a wave reads 1 KiB contiguously.
template <int U, int kElems>
__global__ __launch_bounds__(kTile) void token_cat_fp8_kernel(TokenCatArgs a) {
    const int64_t row = blockIdx.x;
    const int64_t cols = a.a_cols + a.b_cols;
    const int cpr = (int)(cols / kElems);
    const int a_chunks = (int)(a.a_cols / kElems);
    const float inv = 1.0f / *a.scale;  // IEEE division
    float f[U][kElems];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int c = (blockIdx.y * U + u) * kTile + threadIdx.x;
        if (c >= cpr) continue;
        const uint16_t* src = c < a_chunks ? a.a + row * a.a_cols + kElems * c
                                           : a.b + row * a.b_cols + kElems * (c - a_chunks);
#pragma unroll
        for (int h = 0; h < kElems / 8; ++h) {
            float t[8];
            unpack8(stream_load16(src + 8 * h), t);
#pragma unroll
            for (int e = 0; e < 8; ++e) f[u][8 * h + e] = t[e];
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int c = (blockIdx.y * U + u) * kTile + threadIdx.x;
        if (c >= cpr) continue;
        uint32_t w[kElems / 4];
#pragma unroll
        for (int q = 0; q < kElems / 4; ++q)
            w[q] = pack_e4m3x4(clamp_e4m3(f[u][4 * q] * inv), clamp_e4m3(f[u][4 * q + 1] * inv),
                               clamp_e4m3(f[u][4 * q + 2] * inv), clamp_e4m3(f[u][4 * q + 3] * inv));
        uint8_t* dst = a.out + row * cols + kElems * c;
        if (kElems == 16) store16(dst, (u32x4){w[0], w[1], w[2], w[3]});
        else store8(dst, (u32x2){w[0], w[1]});
    }
}

// FP4 with two lanes per 16-element group: lane 2g + h holds elements 8h..8h+7
// of group g (one 16-byte load; a wave reads 1 KiB contiguously); the group
// maximum is exchanged between the two lanes with one DPP step, both lanes
// derive the same scale, each writes 4 packed bytes, the even lane the scale.
__global__ __launch_bounds__(kTile) void token_cat_fp4_pair_kernel(TokenCatArgs a) {
    const int64_t row = blockIdx.x;  // < round_up(rows, 128)
    const int64_t cols = a.a_cols + a.b_cols;
    const int groups = (int)(cols >> 4);
    const int half = (int)(blockIdx.y * kTile + threadIdx.x);  // 8-element half-group
    const int g = half >> 1;
    const int h = half & 1;
    const bool live = g < groups;  // whole pairs only: groups * 2 halves
    if (row >= a.rows) {  // pad rows of the scale matrix
        if (live && h == 0) a.out_scales[row * groups + g] = 0;
        return;
    }
    const float gscale = *a.scale;  // global inverse scale
    const int a_groups = (int)(a.a_cols >> 4);
    float f[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (live) {
        const uint16_t* src = g < a_groups ? a.a + row * a.a_cols + 16 * g + 8 * h
                                           : a.b + row * a.b_cols + 16 * (g - a_groups) + 8 * h;
        unpack8(stream_load16(src), f);
    }
    float amax = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = __builtin_fmaxf(amax, __builtin_fabsf(f[e]));
    const float other = __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, amax), 0xB1, 0xF, 0xF, false));
    amax = __builtin_fmaxf(amax, other);  // lanes 2g and 2g + 1 exchange (quad_perm [1,0,3,2])
    if (!live) return;
    const float s_pre = (amax / 6.0f) * gscale;
    const uint32_t s8 =
        (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(__builtin_fminf(s_pre, 448.0f), 0.0f, 0, false) & 0xFFu;
    uint32_t packed = 0;
    if (s8 != 0) {
        const float kq = gscale / e4m3_value_pos(s8);  // IEEE division
        float t[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) t[e] = f[e] * kq;
        packed = pack_e2m1x8(t);
    }
    store4(a.out + row * (cols >> 1) + 8 * g + 4 * h, packed);
    if (h == 0) a.out_scales[row * groups + g] = (uint8_t)s8;
}

__global__ __launch_bounds__(kTile) void token_cat_fp4_kernel(TokenCatArgs a) {
    const int64_t row = blockIdx.x;  // < round_up(rows, 128)
    const int64_t cols = a.a_cols + a.b_cols;
    const int groups = (int)(cols >> 4);
    const int g = blockIdx.y * kTile + threadIdx.x;
    if (g >= groups) return;
    uint8_t* scale_out = a.out_scales + row * groups + g;
    if (row >= a.rows) {  // pad rows of the scale matrix
        *scale_out = 0;
        return;
    }
    const float gscale = *a.scale;  // global inverse scale
    float f[16];
    load16x2(cat_source(a, row, g), f);
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
    store8(a.out + row * (cols >> 1) + 8 * g, packed);
    *scale_out = (uint8_t)s8;
}

template <int U, int kElems>
hipError_t launch_fp8_u(const TokenCatArgs& a, hipStream_t stream) {
    const int64_t chunks = (a.a_cols + a.b_cols) / kElems;
    const dim3 grid((unsigned)a.rows, (unsigned)((chunks + U * kTile - 1) / (U * kTile)));
    hipLaunchKernelGGL((token_cat_fp8_kernel<U, kElems>), grid, dim3(kTile), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_fp4_pair(const TokenCatArgs& a, hipStream_t stream) {
    const int64_t rows_padded = (a.rows + 127) / 128 * 128;
    const int64_t halves = (a.a_cols + a.b_cols) / 8;
    const dim3 grid((unsigned)rows_padded, (unsigned)((halves + kTile - 1) / kTile));
    hipLaunchKernelGGL(token_cat_fp4_pair_kernel, grid, dim3(kTile), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

// 8 elements per lane, two chunks per thread: measured best on MI355X at
// 4608 x (6144 + 18432) (~75% of HBM peak).
hipError_t launch_token_cat_fp8(const TokenCatArgs& a, hipStream_t stream) {
    return launch_fp8_u<2, 8>(a, stream);
}

// One lane per 16-element group measured faster than two lanes per group.
hipError_t launch_token_cat_fp4(const TokenCatArgs& a, hipStream_t stream) {
    const int64_t rows_padded = (a.rows + 127) / 128 * 128;
    const int64_t groups = (a.a_cols + a.b_cols) / 16;
    const dim3 grid((unsigned)rows_padded, (unsigned)((groups + kTile - 1) / kTile));
    hipLaunchKernelGGL(token_cat_fp4_kernel, grid, dim3(kTile), 0, stream, a);
    return hipGetLastError();
}

}  // namespace dit

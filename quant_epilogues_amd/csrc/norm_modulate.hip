// norm_modulate.hip -- LayerNorm (no affine) + AdaLN scale/shift + static FP8
// E4M3 quantisation with dual bf16 + FP8 output, optionally preceded by an
// input bias and a gated residual that is written out as well.
//
// What is computed follows the sglang PR 37156 page (norm_scale_shift excerpt
// under "Key source snippets": bf16 norm, y = bf16(norm * (1 + scale) +
// shift), q = e4m3(clamp(y * (1/input_scale)))) and the sglang PR 37116 page
// ("Implementation breakdown" item 3: x + bias folded into the gated-residual
// norm kernel).
//
// Layout on gfx950: one wave64 per row. A row of `hidden` bf16 is cut into
// 16-byte chunks; lane l holds chunks l, l + 64, l + 128, ... (V of them), so
// each load or store instruction of the wave moves 1 KiB of contiguous HBM.
// The whole row stays in registers between the statistics and the outputs.
// Row statistics are accumulated in binary64 and reduced with DPP within
// 16-lane rows, then across rows.
#include "dit_device.h"
#include "kernels.h"

namespace dit {
namespace {

enum Mode : int { kPlain = 0, kResidual = 1, kBiasResidual = 2 };

template <int V, int MODE>
__global__ __launch_bounds__(256) void norm_modulate_fp8_kernel(NormModulateArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= a.rows) return;
    const int cpr = a.hidden >> 3;  // 16-byte chunks per row
    const int64_t base = row * (int64_t)a.hidden;

    // Chunk k of this lane is column chunk c = lane + 64 k. Only the last one
    // can fall beyond the row (V = ceil(cpr / 64)).
    u32x4 xin[V];
    u32x4 rin[V];
#pragma unroll
    for (int k = 0; k < V; ++k) {
        const int c = lane + 64 * k;
        const bool ok = (k < V - 1) || (c < cpr);
        xin[k] = ok ? load16(a.x + base + 8 * c) : (u32x4){0, 0, 0, 0};
        if (MODE != kPlain) rin[k] = ok ? load16(a.residual + base + 8 * c) : (u32x4){0, 0, 0, 0};
    }

    // v: the row to normalise (x, or the new residual).
    float v[V][8];
#pragma unroll
    for (int k = 0; k < V; ++k) {
        const int c = lane + 64 * k;
        const bool ok = (k < V - 1) || (c < cpr);
        if (MODE == kPlain) {
            unpack8(xin[k], v[k]);
        } else {
            float xf[8], rf[8], gf[8];
            unpack8(xin[k], xf);
            unpack8(rin[k], rf);
            unpack8(ok ? load16(a.gate + 8 * c) : (u32x4){0, 0, 0, 0}, gf);
            if (MODE == kBiasResidual) {
                float bf[8];
                unpack8(ok ? load16(a.bias + 8 * c) : (u32x4){0, 0, 0, 0}, bf);
#pragma unroll
                for (int i = 0; i < 8; i += 2) {  // xb = bf16(x + bias)
                    const uint32_t w = pack_bf16(xf[i] + bf[i], xf[i + 1] + bf[i + 1]);
                    xf[i] = bf_lo(w);
                    xf[i + 1] = bf_hi(w);
                }
            }
            uint32_t rw[4];
#pragma unroll
            for (int i = 0; i < 8; i += 2) {
                // gate * xb is exact in fp32 (8 x 8 significant bits); the sum
                // with the residual is rounded once to bf16.
                const uint32_t lo = bf16_bits_exact_sum(gf[i] * xf[i], rf[i]);
                const uint32_t hi = bf16_bits_exact_sum(gf[i + 1] * xf[i + 1], rf[i + 1]);
                rw[i / 2] = lo | (hi << 16);
                v[k][i] = bf_lo(lo);
                v[k][i + 1] = bf_lo(hi);
            }
            if (ok) store16(a.r_out + base + 8 * c, (u32x4){rw[0], rw[1], rw[2], rw[3]});
        }
    }

    // Mean and biased variance from one pass of binary64 sums. The square of
    // a bf16 value is exact, so both sums are exact for ordinary rows and
    // var = E[v^2] - mean^2 is within a few binary64 ulps of the two-pass
    // value unless |mean| dwarfs the spread by many orders of magnitude.
    double s1 = 0.0, s2 = 0.0;
#pragma unroll
    for (int k = 0; k < V; ++k) {
        const bool ok = (k < V - 1) || (lane + 64 * k < cpr);
        if (ok) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const double d = (double)v[k][i];
                s1 += d;
                s2 = __builtin_fma(d, d, s2);
            }
        }
    }
    s1 = wave_sum(s1);
    s2 = wave_sum(s2);
    const double mean = s1 / (double)a.hidden;
    const double var = __builtin_fmax(s2 / (double)a.hidden - mean * mean, 0.0);
    const float factor = (float)(1.0 / __builtin_sqrt(var + (double)a.eps));
    const float mean32 = (float)mean;
    const float inv = 1.0f / *a.input_scale;  // IEEE division

#pragma unroll
    for (int k = 0; k < V; ++k) {
        const int c = lane + 64 * k;
        const bool ok = (k < V - 1) || (c < cpr);
        if (!ok) continue;
        float sc[8], sh[8];
        unpack8(load16(a.scale + 8 * c), sc);
        unpack8(load16(a.shift + 8 * c), sh);
        uint32_t yw[4];
        float yv[8];
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
            const float t0 = (v[k][i] - mean32) * factor;
            const float t1 = (v[k][i + 1] - mean32) * factor;
            const uint32_t nw = pack_bf16(t0, t1);  // normalised row, bf16
            const float m0 = __builtin_fmaf(bf_lo(nw), 1.0f + sc[i], sh[i]);
            const float m1 = __builtin_fmaf(bf_hi(nw), 1.0f + sc[i + 1], sh[i + 1]);
            yw[i / 2] = pack_bf16(m0, m1);
            yv[i] = bf_lo(yw[i / 2]);
            yv[i + 1] = bf_hi(yw[i / 2]);
        }
        const uint32_t q0 = pack_e4m3x4(clamp_e4m3(yv[0] * inv), clamp_e4m3(yv[1] * inv),
                                        clamp_e4m3(yv[2] * inv), clamp_e4m3(yv[3] * inv));
        const uint32_t q1 = pack_e4m3x4(clamp_e4m3(yv[4] * inv), clamp_e4m3(yv[5] * inv),
                                        clamp_e4m3(yv[6] * inv), clamp_e4m3(yv[7] * inv));
        store16(a.y + base + 8 * c, (u32x4){yw[0], yw[1], yw[2], yw[3]});
        store8(a.q + base + 8 * c, (u32x2){q0, q1});
    }
}

template <int MODE>
hipError_t launch_mode(const NormModulateArgs& a, hipStream_t stream) {
    const int cpr = a.hidden / 8;
    const int V = (cpr + 63) / 64;
    const dim3 grid((unsigned)((a.rows + 3) / 4));
    const dim3 block(256);
#define DIT_NM_CASE(VV)                                                              \
    case VV:                                                                         \
        hipLaunchKernelGGL((norm_modulate_fp8_kernel<VV, MODE>), grid, block, 0, stream, a); \
        break;
    switch (V) {
        DIT_NM_CASE(1) DIT_NM_CASE(2) DIT_NM_CASE(3) DIT_NM_CASE(4)
        DIT_NM_CASE(5) DIT_NM_CASE(6) DIT_NM_CASE(7) DIT_NM_CASE(8)
        DIT_NM_CASE(9) DIT_NM_CASE(10) DIT_NM_CASE(11) DIT_NM_CASE(12)
        default: return hipErrorInvalidValue;
    }
#undef DIT_NM_CASE
    return hipGetLastError();
}

}  // namespace

hipError_t launch_norm_modulate_fp8(const NormModulateArgs& a, hipStream_t stream) {
    if (a.residual == nullptr) return launch_mode<kPlain>(a, stream);
    if (a.bias == nullptr) return launch_mode<kResidual>(a, stream);
    return launch_mode<kBiasResidual>(a, stream);
}

}  // namespace dit

// bias_mul_add.hip -- final gated residual with an absorbed output bias:
// y = bf16(bf16(x + bias) * gate + residual), the multiply-add rounded once.
//
// What is computed follows the sglang PR 37116 page (the bias_mul_add excerpt
// under "Key source snippets" and the review highlights): the bias add is
// rounded to bf16, and the multiply-add is a native bf16 FMA, i.e. one
// rounding; routing it through fp32 and then bf16 would round twice and break
// product ties at large magnitudes.
//
// On gfx950 the product of two bf16 values is exact in fp32, so only the final
// sum needs care: pack8_exact_sum rounds p + residual once.
//
// Layout: WPR waves per row and RPW rows per workgroup; wave w of a row takes
// 16-byte chunks 64 (w + WPR k) + lane for k < V (rows wider than
// 512 * WPR * V columns loop), so each instruction of a wave moves 1 KiB of
// contiguous HBM. x and residual stream through with non-temporal loads;
// bias and gate are row-broadcast and stay in L2.
#include "dit_device.h"
#include "kernels.h"

namespace dit {
namespace {

template <bool kHasBias, int WPR, int RPW, int V>
__global__ __launch_bounds__(64 * WPR * RPW) void bias_mul_add_kernel(BiasMulAddArgs a) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int sw = wave % WPR;
    const int64_t row = (int64_t)blockIdx.x * RPW + wave / WPR;
    if (row >= a.rows) return;
    const int cpr = (int)(a.hidden >> 3);
    const int64_t base = row * a.hidden;
    for (int c0 = 0; c0 < cpr; c0 += 64 * WPR * V) {
        u32x4 xv[V], rv[V];
#pragma unroll
        for (int k = 0; k < V; ++k) {
            const int c = c0 + 64 * (sw + WPR * k) + lane;
            if (c < cpr) {
                xv[k] = stream_load16(a.x + base + 8 * c);
                rv[k] = stream_load16(a.residual + base + 8 * c);
            }
        }
#pragma unroll
        for (int k = 0; k < V; ++k) {
            const int c = c0 + 64 * (sw + WPR * k) + lane;
            if (c >= cpr) continue;
            float xf[8], rf[8], gf[8];
            unpack8(xv[k], xf);
            unpack8(rv[k], rf);
            unpack8(load16(a.gate + 8 * c), gf);
            if (kHasBias) {
                float bf[8];
                unpack8(load16(a.bias + 8 * c), bf);
#pragma unroll
                for (int i = 0; i < 8; i += 2) {  // b = bf16(x + bias)
                    const uint32_t w = pack_bf16(xf[i] + bf[i], xf[i + 1] + bf[i + 1]);
                    xf[i] = bf_lo(w);
                    xf[i + 1] = bf_hi(w);
                }
            }
            float prod[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) prod[i] = xf[i] * gf[i];  // exact in fp32
            uint32_t yw[4];
            pack8_exact_sum(prod, rf, yw);
            store16(a.y + base + 8 * c, (u32x4){yw[0], yw[1], yw[2], yw[3]});
        }
    }
}

template <bool kHasBias, int WPR, int RPW, int V>
hipError_t launch_geom(const BiasMulAddArgs& a, hipStream_t stream) {
    const uint64_t blocks = (uint64_t)((a.rows + RPW - 1) / RPW);
    if (blocks * (64 * WPR * RPW) >= kMaxGridLanes) return kGridTooLarge;
    hipLaunchKernelGGL((bias_mul_add_kernel<kHasBias, WPR, RPW, V>), dim3((unsigned)blocks),
                       dim3(64 * WPR * RPW), 0, stream, a);
    return hipGetLastError();
}

// Six waves per row, one chunk per lane (measured best on MI355X at hidden
// 3072: 384 chunks = one pass; wider rows loop).
template <bool kHasBias>
hipError_t launch_bias(const BiasMulAddArgs& a, hipStream_t stream) {
    return launch_geom<kHasBias, 6, 1, 1>(a, stream);
}

}  // namespace

hipError_t launch_bias_mul_add(const BiasMulAddArgs& a, hipStream_t stream) {
    return a.bias ? launch_bias<true>(a, stream) : launch_bias<false>(a, stream);
}

}  // namespace dit

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
// sum needs care: bf16_bits_exact_sum rounds p + residual once.
//
// Layout: one wave64 per row; lane l handles 16-byte chunks l, l + 64, ...,
// processed kUnroll chunks at a time so that 2 * kUnroll 16-byte loads per lane
// are in flight. bias and gate are row-broadcast and stay in L2.
#include "dit_device.h"
#include "kernels.h"

namespace dit {
namespace {

constexpr int kUnroll = 6;

template <bool kHasBias>
__global__ __launch_bounds__(256) void bias_mul_add_kernel(BiasMulAddArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= a.rows) return;
    const int cpr = (int)(a.hidden >> 3);
    const int64_t base = row * a.hidden;

    for (int c0 = 0; c0 < cpr; c0 += 64 * kUnroll) {
        u32x4 xv[kUnroll], rv[kUnroll];
#pragma unroll
        for (int k = 0; k < kUnroll; ++k) {
            const int c = c0 + lane + 64 * k;
            if (c < cpr) {
                xv[k] = load16(a.x + base + 8 * c);
                rv[k] = load16(a.residual + base + 8 * c);
            }
        }
#pragma unroll
        for (int k = 0; k < kUnroll; ++k) {
            const int c = c0 + lane + 64 * k;
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
            uint32_t yw[4];
#pragma unroll
            for (int i = 0; i < 8; i += 2) {
                const uint32_t lo = bf16_bits_exact_sum(xf[i] * gf[i], rf[i]);
                const uint32_t hi = bf16_bits_exact_sum(xf[i + 1] * gf[i + 1], rf[i + 1]);
                yw[i / 2] = lo | (hi << 16);
            }
            store16(a.y + base + 8 * c, (u32x4){yw[0], yw[1], yw[2], yw[3]});
        }
    }
}

}  // namespace

hipError_t launch_bias_mul_add(const BiasMulAddArgs& a, hipStream_t stream) {
    const dim3 grid((unsigned)((a.rows + 3) / 4));
    if (a.bias)
        hipLaunchKernelGGL(bias_mul_add_kernel<true>, grid, dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL(bias_mul_add_kernel<false>, grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace dit

// bias_mul_add.hip -- final gated residual with an absorbed output bias:
// y = bf16(bf16(x + bias) * gate + residual), the multiply-add rounded once.
//
// What is computed follows the sglang PR 37116 page (the bias_mul_add excerpt
// under "Key source snippets" and the review highlights): the bias add is
// rounded to bf16, and the multiply-add is a native bf16 FMA, i.e. one
// rounding; routing it through fp32 and then bf16 would round twice and break
// product ties at large magnitudes.
//
// On gfx950 the product of two bf16 values is exact in fp32 (below 2^128 in
// magnitude, the library's input domain), so only the final sum needs care:
// pack8_exact_sum rounds p + residual once.
//
// Layout: one wave64 per workgroup, one 64-chunk segment of a row per wave;
// lane t of segment s takes the 16-byte chunk 64 s + t of its row, so each
// instruction of a wave moves 1 KiB of contiguous HBM and consecutive
// workgroups (segments of a row, then the next row) sweep memory in address
// order. One-wave workgroups are dispatched and retired independently; on
// MI355X they streamed this shape 6% faster than one six-wave workgroup per
// row. x and residual stream through with non-temporal loads; bias and gate
// are row-broadcast and stay in L2.
#include "dit_device.h"
#include "kernels.h"

namespace dit {
namespace {

constexpr int kThreads = 64;  // one wave, one 64-chunk (512-column) segment of a row

template <bool kHasBias>
__global__ __launch_bounds__(kThreads) void bias_mul_add_kernel(BiasMulAddArgs a, int segs) {
    const int64_t row = blockIdx.x / (unsigned)segs;
    const int c = (int)(blockIdx.x % (unsigned)segs) * kThreads + (int)threadIdx.x;
    const int cpr = (int)(a.hidden >> 3);
    const uint16_t* xrow = a.x + row * a.hidden;
    const uint16_t* rrow = a.residual + row * a.hidden;
    uint16_t* yrow = a.y + row * a.hidden;
    if (c < cpr) {
        // All four loads are issued before any of them is used: the
        // scheduling barrier keeps the compiler from waiting on the gate's
        // L2 round trip before it issues the bias load.
        const u32x4 xv = stream_load16(xrow + 8 * c);
        const u32x4 rv = stream_load16(rrow + 8 * c);
        const u32x4 gv = load16(a.gate + 8 * c);
        const u32x4 bv = kHasBias ? load16(a.bias + 8 * c) : (u32x4){0u, 0u, 0u, 0u};
        __builtin_amdgcn_sched_barrier(0);
        float xf[8], rf[8], gf[8];
        unpack8(gv, gf);
        if (kHasBias) {
            float bf[8];
            unpack8(bv, bf);
            unpack8(xv, xf);
#pragma unroll
            for (int i = 0; i < 8; i += 2) {  // b = bf16(x + bias)
                const uint32_t w = pack_bf16(xf[i] + bf[i], xf[i + 1] + bf[i + 1]);
                xf[i] = bf_lo(w);
                xf[i + 1] = bf_hi(w);
            }
        } else {
            unpack8(xv, xf);
        }
        unpack8(rv, rf);
        float prod[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) prod[i] = xf[i] * gf[i];  // exact in fp32 below 2^128
        uint32_t yw[4];
        pack8_exact_sum(prod, rf, yw);
        store16(yrow + 8 * c, (u32x4){yw[0], yw[1], yw[2], yw[3]});
    }
}

template <bool kHasBias>
hipError_t launch_bias(const BiasMulAddArgs& a, hipStream_t stream) {
    const int segs = (int)(((a.hidden >> 3) + kThreads - 1) / kThreads);  // segments per row
    const uint64_t blocks = (uint64_t)a.rows * (uint64_t)segs;
    if (blocks * kThreads >= kMaxGridLanes) return kGridTooLarge;
    hipLaunchKernelGGL(bias_mul_add_kernel<kHasBias>, dim3((unsigned)blocks), dim3(kThreads), 0,
                       stream, a, segs);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bias_mul_add(const BiasMulAddArgs& a, hipStream_t stream) {
    return a.bias ? launch_bias<true>(a, stream) : launch_bias<false>(a, stream);
}

}  // namespace dit

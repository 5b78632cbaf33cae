// qkv_epilogue.hip -- per-head RMSNorm of Q and K, interleaved RoPE, V copy and
// the joint [text, image] packing, read straight from the packed QKV GEMM
// output through strided views.
//
// What is computed follows the sglang PR 37123 page ("Implementation
// breakdown" items 3-4 and the forward excerpt under "Key source snippets"):
// Q/K of each stream are RMS-normalised per head with that stream's weight and
// epsilon, rotated by interleaved (non-NeoX) RoPE from an fp32 cache, V is
// copied, and all three are written in [text, image] order.
//
// Layout on gfx950: one wave64 per (joint token, part in {Q, K}, group of
// kPasses * 4 heads), and one per (joint token, group of 4 heads) for the V
// copy. The wave is four 16-lane rows; row r takes heads r, r + 4, ... of its
// group, and lane s of a row holds elements 8s..8s+7 of its head (one 16-byte
// load). A head's sum of squares is a 16-lane DPP
// reduction, the RoPE pairs (2i, 2i+1) sit inside one lane, and the lane's
// four cos/sin values are loaded once per wave.
//
// Rounding: the RMS statistic is binary64; 1/sqrt is refined in binary64 from
// the fp32 seed and rounded once to fp32; the normalised head is rounded to
// bf16 before RoPE; each RoPE output is one binary64 fma of exact products,
// rounded to bf16.
#include "dit_device.h"
#include "kernels.h"

namespace dit {
namespace {

// bf16 bits (round to nearest even) of the binary64 value d, given its fp32
// rounding f, when f lies exactly on a bf16 midpoint: RN32 cannot carry a
// value across a midpoint, only onto one, so d decides the side and an exact
// tie keeps the even neighbour.
__device__ __forceinline__ uint32_t bf16_of_midpoint(float f, double d) {
    const uint32_t t = __float_as_uint(f) >> 16;  // f truncated to bf16 (toward zero)
    if (d == (double)f) return t + (t & 1u);      // exact tie: the even neighbour
    return t + (__builtin_fabs(d) > __builtin_fabs((double)f) ? 1u : 0u);
}

// Interleaved RoPE of one lane's 8 normalised values (pairs (2q, 2q + 1)),
// each output one binary64 fma of exact products (a bf16 value times an fp32
// table entry), rounded to bf16 through fp32. A value whose fp32 rounding
// sits on a bf16 midpoint (one wave-uniform branch, almost never taken) is
// recomputed and settled from binary64, so no binary64 value has to outlive
// its conversion.
__device__ __forceinline__ void rope_pack8(const float (&n)[8], const float (&cs)[4],
                                           const float (&sn)[4], uint32_t (&w)[4]) {
    bool tie = false;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const double n0 = (double)n[2 * q], n1 = (double)n[2 * q + 1];
        const double c = (double)cs[q], sv = (double)sn[q];
        const float f0 = (float)__builtin_fma(n0, c, -(n1 * sv));
        const float f1 = (float)__builtin_fma(n1, c, n0 * sv);
        tie |= (__float_as_uint(f0) & 0xFFFFu) == 0x8000u;
        tie |= (__float_as_uint(f1) & 0xFFFFu) == 0x8000u;
        w[q] = pack_bf16(f0, f1);
    }
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(tie) != 0, 0)) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const double n0 = (double)n[2 * q], n1 = (double)n[2 * q + 1];
            const double c = (double)cs[q], sv = (double)sn[q];
            const double d0 = __builtin_fma(n0, c, -(n1 * sv));
            const double d1 = __builtin_fma(n1, c, n0 * sv);
            const float f0 = (float)d0, f1 = (float)d1;
            if ((__float_as_uint(f0) & 0xFFFFu) == 0x8000u)
                w[q] = (w[q] & 0xFFFF0000u) | bf16_of_midpoint(f0, d0);
            if ((__float_as_uint(f1) & 0xFFFFu) == 0x8000u)
                w[q] = (w[q] & 0x0000FFFFu) | (bf16_of_midpoint(f1, d1) << 16);
        }
    }
}

// kPasses 4-head passes per Q/K wave (a wave covers 4 * kPasses heads); a
// token has kHBlocks such head groups, and a unit is one of them. One wave per
// workgroup; the 1-D grid holds the Q units, then the K units, then kPasses V
// waves per unit, each copying one 4-head pass (a single 16-byte chunk per
// lane, the form a plain copy streams best in: 2.5% faster over the launch
// than V waves of 4 * kPasses heads). Unit u is head group u % kHBlocks of
// joint token u / kHBlocks, so consecutive waves read consecutive memory.
// One-wave workgroups are dispatched and retired independently; on MI355X
// they ran this shape 1.5% faster than four-wave workgroups. Everything
// derived from the workgroup index (token, stream, source and weight
// pointers) is wave-uniform and lives in scalar registers: the pointers come
// from scalar loads of the argument block, so the streaming loads issue
// without waiting on per-lane loads.
template <int kPasses, int kHBlocks>
__global__ __launch_bounds__(64) void qkv_epilogue_kernel(QkvArgs a) {
    constexpr int kHeadsPerWave = 4 * kPasses;
    const int lane = threadIdx.x;
    const int r = lane >> 4;  // head slot within a pass
    const int s = lane & 15;  // 8-element slice of the head
    const uint64_t units = (uint64_t)(a.txt_rows + a.img_rows) * kHBlocks;
    const uint64_t b = blockIdx.x;
    if (b >= 2 * units) {  // V: a bit copy of one 4-head pass into the joint layout
        const uint64_t vb = b - 2 * units;
        const uint64_t unit = vb / kPasses;
        const int p = (int)(vb % kPasses);
        const int64_t j = (int64_t)(unit / kHBlocks);
        const int hb = (int)(unit % kHBlocks);
        const bool is_txt = j < a.txt_rows;
        const int64_t i = is_txt ? j : j - a.txt_rows;
        const uint16_t* src = (is_txt ? a.txt[2] : a.img[2]) + i * (is_txt ? a.txt_stride : a.img_stride);
        uint16_t* dst = a.joint[2] + j * (int64_t)a.heads * kHeadDim;
        const int head = hb * kHeadsPerWave + 4 * p + r;
        if (head < a.heads)
            store16(dst + head * kHeadDim + 8 * s, stream_load16(src + head * kHeadDim + 8 * s));
        return;
    }
    const int part = (int)(b / units);  // 0 = Q, 1 = K
    const uint64_t unit = b % units;
    const int64_t j = (int64_t)(unit / kHBlocks);
    const int hb = (int)(unit % kHBlocks);

    const bool is_txt = j < a.txt_rows;
    const int64_t i = is_txt ? j : j - a.txt_rows;
    const uint16_t* src = (is_txt ? a.txt[part] : a.img[part]) +
                          i * (is_txt ? a.txt_stride : a.img_stride);
    uint16_t* dst = a.joint[part] + j * (int64_t)a.heads * kHeadDim;

    // Head slots past the last head (heads not a multiple of 4 * kPasses)
    // load the last head again, compute on it (the 16-lane row reduction
    // never mixes rows) and skip their store: every load is unconditional.
    int head[kPasses];
    u32x4 xin[kPasses];
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
        head[p] = hb * kHeadsPerWave + 4 * p + r;
        const int hl = head[p] < a.heads ? head[p] : a.heads - 1;
        xin[p] = stream_load16(src + hl * kHeadDim + 8 * s);
    }

    float w[8];
    unpack8(load16((is_txt ? a.txt_w[part] : a.img_w[part]) + 8 * s), w);
    const float* cos_row = (is_txt ? a.txt_cos : a.img_cos) + i * a.rope_stride + 4 * s;
    const float* sin_row = (is_txt ? a.txt_sin : a.img_sin) + i * a.rope_stride + 4 * s;
    const float4 c4 = *reinterpret_cast<const float4*>(cos_row);
    const float4 s4 = *reinterpret_cast<const float4*>(sin_row);
    const float cs[4] = {c4.x, c4.y, c4.z, c4.w};
    const float sn[4] = {s4.x, s4.y, s4.z, s4.w};
    const double eps = (double)(is_txt ? a.txt_eps : a.img_eps);

#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
        float x[8];
        unpack8(xin[p], x);
        double ss = 0.0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const double d = (double)x[e];
            ss = __builtin_fma(d, d, ss);  // bf16 squares are exact
        }
        ss = row16_sum(ss);
        const float inv = rsqrt_rn32(ss * (1.0 / kHeadDim) + eps);

        float n[8];  // the normalised head, rounded to bf16
#pragma unroll
        for (int e = 0; e < 8; ++e) n[e] = round_bf16((x[e] * inv) * w[e]);
        uint32_t ow[4];
        rope_pack8(n, cs, sn, ow);
        if (head[p] < a.heads)
            store16(dst + head[p] * kHeadDim + 8 * s, (u32x4){ow[0], ow[1], ow[2], ow[3]});
    }
}

template <int kPasses, int kHBlocks>
hipError_t launch_groups(const QkvArgs& a, hipStream_t stream) {
    const uint64_t units = (uint64_t)(a.txt_rows + a.img_rows) * kHBlocks;
    const uint64_t blocks = units * (2 + kPasses);  // Q and K units, then kPasses V waves per unit
    if (blocks * 64 >= kMaxGridLanes) return kGridTooLarge;
    hipLaunchKernelGGL((qkv_epilogue_kernel<kPasses, kHBlocks>), dim3((unsigned)blocks), dim3(64), 0,
                       stream, a);
    return hipGetLastError();
}

template <int kPasses>
hipError_t launch_passes(const QkvArgs& a, hipStream_t stream) {
    static_assert(kMaxHeads <= 6 * 4 * kPasses, "head groups beyond six need an instance");
    switch ((a.heads + 4 * kPasses - 1) / (4 * kPasses)) {
        case 1: return launch_groups<kPasses, 1>(a, stream);
        case 2: return launch_groups<kPasses, 2>(a, stream);
        case 3: return launch_groups<kPasses, 3>(a, stream);
        case 4: return launch_groups<kPasses, 4>(a, stream);
        case 5: return launch_groups<kPasses, 5>(a, stream);
        default: return launch_groups<kPasses, 6>(a, stream);
    }
}

}  // namespace

// Three passes (12 heads per wave) measured best on MI355X at 24 and 48
// heads x 128 with one-wave workgroups: 2.5% faster than six passes, 1.5%
// faster than two.
hipError_t launch_qkv_epilogue(const QkvArgs& a, hipStream_t stream) {
    return launch_passes<kQkvHeadsPerWave / 4>(a, stream);
}

}  // namespace dit

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
// Layout on gfx950: a row of `hidden` bf16 is cut into 16-byte chunks (8
// values) and owned by WPR waves; wave w of the row takes chunks
// 64 (w + WPR k) + lane for k < V, so each load or store instruction of a wave
// moves 1 KiB of contiguous HBM. A workgroup holds RPW rows; it first issues
// its streaming loads, then (when they fit in 48 KiB, kLds) converts the
// row-broadcast vectors once into fp32 in LDS (1 + scale, shift, and gate,
// bias for the residual variants), which takes those conversions off the
// per-element path; otherwise each wave reads them from L2. The row stays in
// registers between the statistics and the outputs. Statistics are binary64:
// DPP/shuffle within each wave, then (WPR > 1) the wave partials through LDS,
// added in wave order so every thread of the row agrees bit for bit.
#include "dit_device.h"
#include "kernels.h"

namespace dit {
namespace {

enum Mode : int { kPlain = 0, kResidual = 1, kBiasResidual = 2 };

// Number of fp32 column vectors staged in LDS per mode.
template <int MODE>
constexpr int kColVecs = MODE == kPlain ? 2 : (MODE == kResidual ? 3 : 4);

__device__ __forceinline__ void lds_read8(const float* p, float (&f)[8]) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
    f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}

__device__ __forceinline__ void lds_write8(float* p, const float (&f)[8]) {
    *reinterpret_cast<float4*>(p) = make_float4(f[0], f[1], f[2], f[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(f[4], f[5], f[6], f[7]);
}

constexpr size_t kLdsColsMax = 48 * 1024;  // bytes of fp32 column vectors staged in LDS

// The 8 fp32 column values of chunk c of column vector `which` (0: 1 + scale,
// 1: shift, 2: gate, 3: bias), from LDS or from the bf16 vector in memory.
template <bool kLds>
__device__ __forceinline__ void col8(const float* cols, const NormModulateArgs& a, int which,
                                     int c, float (&f)[8]) {
    if (kLds) {
        lds_read8(cols + (size_t)which * a.hidden + 8 * c, f);
        return;
    }
    const uint16_t* src = which == 0 ? a.scale : which == 1 ? a.shift : which == 2 ? a.gate : a.bias;
    unpack8(load16(src + 8 * c), f);
    if (which == 0) {
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = 1.0f + f[i];
    }
}

// kExact (plain variant only): hidden == 512 WPR V, so every chunk index lies
// inside the row and no load needs a predicate; a wave past the last row then
// reads the last row again (its results are dropped) instead of zero-filling
// its registers. For the residual variants the predicated form measured
// faster on MI355X and is kept.
// kHoist (latency-bound launches, few rows): the column vectors are loaded
// together with the row instead of after the statistics, which takes their
// L2 round trips off the critical path; it costs registers, which only matter
// when many rows are in flight.
// kStage (plain variant, RPW >= 2, no kLds / kHoist): the waves of the first
// row slot load their chunks of scale and shift before their row loads and
// park the raw bf16 in LDS (2 x 16 bytes per chunk and lane); the barrier of
// the cross-wave reduction makes them visible to every row slot, which reads
// them back after the statistics instead of waiting on an L2 round trip
// there. The registers they pass through are free again before the row is
// converted, so occupancy stays where the streaming loads put it.
// A launch covers one or two independent row sets (streams) that share the
// width and the kernel instance: workgroups [0, blocks0) take the rows of a0,
// the rest those of a1 (Qwen-Image's image and text rows, each with its own
// modulation vectors, FP8 scale and epsilon). The choice is per workgroup, so
// every argument read below is wave-uniform.
// kDual instances (plain variant, FP8 output) serve such two-set launches;
// the others ignore a1 and blocks0.
template <int MODE, int WPR, int RPW, int V, bool kLds, bool kFp4, bool kExact, bool kHoist,
          bool kStage, bool kDual>
__global__ __launch_bounds__(64 * WPR * RPW) void norm_modulate_fp8_kernel(
    NormModulateArgs a0, NormModulateArgs a1, int64_t blocks0, double inv_hidden) {
    // cols: [kColVecs][hidden] fp32 = 1 + scale, shift, gate, bias
    extern __shared__ float cols[];
    __shared__ double scratch[RPW][WPR][2];
    static_assert(!kDual || (MODE == kPlain && !kFp4), "two row sets: plain FP8 variant only");
    NormModulateArgs sel;  // kDual: this workgroup's row set
    if constexpr (kDual) {
        sel = a0;
        if ((int64_t)blockIdx.x >= blocks0) {  // the fields a plain FP8 row reads (wave-uniform)
            sel.y = a1.y;
            sel.q = a1.q;
            sel.x = a1.x;
            sel.scale = a1.scale;
            sel.shift = a1.shift;
            sel.input_scale = a1.input_scale;
            sel.rows = a1.rows;
            sel.eps = a1.eps;
        }
    }
    const NormModulateArgs& a = kDual ? sel : a0;
    const bool second = kDual && (int64_t)blockIdx.x >= blocks0;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int rw = wave / WPR;  // row slot in the workgroup
    const int sw = wave % WPR;  // wave within the row
    const int64_t row = ((int64_t)blockIdx.x - (second ? blocks0 : 0)) * RPW + rw;
    const bool active = row < a.rows;  // wave-uniform; every wave still reaches the barriers
    const int H = a.hidden;
    const int cpr = H >> 3;  // chunks per row
    const int64_t base = row * H;
    const int64_t lbase = (kExact && !active ? a.rows - 1 : row) * H;  // rows >= 1 here

    static_assert(!kStage || (MODE == kPlain && WPR > 1 && RPW >= 2 && !kLds && !kHoist),
                  "kStage needs the plain variant, a cross-wave barrier and no other column path");
    // 0. kStage: column chunks first, so that waiting for them (to write LDS)
    // does not wait for the streaming loads issued after them.
    u32x4* stage = reinterpret_cast<u32x4*>(cols) + (size_t)sw * (2 * V * 64);
    u32x4 cst[kStage ? 2 : 1][V];
    if constexpr (kStage) {
        if (rw == 0) {
#pragma unroll
            for (int k = 0; k < V; ++k) {
                const int c = 64 * (sw + WPR * k) + lane;  // kExact: inside the row
                cst[0][k] = load16(a.scale + 8 * c);
                cst[1][k] = load16(a.shift + 8 * c);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }

    // 1. Streaming loads of this wave's chunks (kHoist: and its column chunks).
    u32x4 xin[V], rin[V], cin[kHoist ? kColVecs<MODE> : 1][V];
    bool ok[V];
#pragma unroll
    for (int k = 0; k < V; ++k) {
        const int c = 64 * (sw + WPR * k) + lane;
        ok[k] = active && (kExact || c < cpr);
        if (kExact) {
            xin[k] = stream_load16(a.x + lbase + 8 * c);
            if (MODE != kPlain) rin[k] = stream_load16(a.residual + lbase + 8 * c);
        } else {
            xin[k] = ok[k] ? stream_load16(a.x + base + 8 * c) : (u32x4){0, 0, 0, 0};
            if (MODE != kPlain)
                rin[k] = ok[k] ? stream_load16(a.residual + base + 8 * c) : (u32x4){0, 0, 0, 0};
        }
    }

    if constexpr (kStage) {
        __builtin_amdgcn_sched_barrier(0);
        if (rw == 0) {
#pragma unroll
            for (int k = 0; k < V; ++k) {
                stage[(0 * V + k) * 64 + lane] = cst[0][k];
                stage[(1 * V + k) * 64 + lane] = cst[1][k];
            }
        }
    }
    if constexpr (kHoist) {
#pragma unroll
        for (int k = 0; k < V; ++k) {
            int c = 64 * (sw + WPR * k) + lane;
            if (!kExact) c = c < cpr ? c : 0;  // columns past the row end are never used
            cin[0][k] = load16(a.scale + 8 * c);
            cin[1][k] = load16(a.shift + 8 * c);
            if (MODE != kPlain) cin[2 % kColVecs<MODE>][k] = load16(a.gate + 8 * c);
            if (MODE == kBiasResidual) cin[3 % kColVecs<MODE>][k] = load16(a.bias + 8 * c);
        }
    }

    const bool want_y = a.y != nullptr, want_q = a.q != nullptr;  // wave-uniform
    const float inv = want_q ? 1.0f / *a.input_scale : 0.0f;  // IEEE division
    const float g4 = kFp4 ? *a.input_scale : 0.0f;  // FP4: the global inverse scale

    // 2. Column vectors to fp32 in LDS, while the streaming loads are in
    // flight; one vector at a time, which keeps the kernel's register peak
    // (and so its occupancy) where the streaming loads alone put it. With FP4
    // output the table g / value(code) of the 126 nonzero E4M3 scale codes
    // follows them (the same IEEE divisions, done once per workgroup).
    float* kq_tab = cols + (size_t)kColVecs<MODE> * H;
    if (kLds) {
        if constexpr (kFp4) {
            for (int code = threadIdx.x; code < 128; code += blockDim.x)
                kq_tab[code] = (code != 0 && code < 127) ? g4 / e4m3_value_pos(code) : 0.0f;
        }
        for (int c = threadIdx.x; c < cpr; c += blockDim.x) {
#pragma unroll 1
            for (int which = 0; which < kColVecs<MODE>; ++which) {
                float f[8];
                col8<false>(cols, a, which, c, f);
                lds_write8(cols + (size_t)which * H + 8 * c, f);
            }
        }
        __syncthreads();
    }

    // 3. The row to normalise: x, or the new residual (0 outside the row).
    float v[V][8];
#pragma unroll
    for (int k = 0; k < V; ++k) {
        const int c = 64 * (sw + WPR * k) + lane;
        if (MODE == kPlain) {
            unpack8(xin[k], v[k]);
            continue;
        }
        float xf[8], rf[8], gf[8];
        unpack8(xin[k], xf);
        unpack8(rin[k], rf);
        // Chunks past the row end must add exactly 0 to the statistics: x and
        // the residual are zero there, and so is the gate.
        if (kExact || ok[k]) {
            if (kHoist) unpack8(cin[2 % kColVecs<MODE>][k], gf);
            else col8<kLds>(cols, a, 2, c, gf);
        } else {
            for (int i = 0; i < 8; ++i) gf[i] = 0.0f;
        }
        if (MODE == kBiasResidual && (kExact || ok[k])) {
            float bf[8];
            if (kHoist) unpack8(cin[3 % kColVecs<MODE>][k], bf);
            else col8<kLds>(cols, a, 3, c, bf);
#pragma unroll
            for (int i = 0; i < 8; i += 2) {  // xb = bf16(x + bias)
                const uint32_t w = pack_bf16(xf[i] + bf[i], xf[i + 1] + bf[i + 1]);
                xf[i] = bf_lo(w);
                xf[i + 1] = bf_hi(w);
            }
        }
        // gate * xb is exact in fp32 (8 x 8 significant bits, below 2^128 in
        // magnitude); the sum with the residual is rounded once to bf16.
        float prod[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) prod[i] = gf[i] * xf[i];
        uint32_t rw4[4];
        pack8_exact_sum(prod, rf, rw4);
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
            v[k][i] = bf_lo(rw4[i / 2]);
            v[k][i + 1] = bf_hi(rw4[i / 2]);
        }
        if (ok[k]) store16(a.r_out + base + 8 * c, (u32x4){rw4[0], rw4[1], rw4[2], rw4[3]});
    }

    // 4. Mean and biased variance from binary64 sums of v and v^2. The square
    // of a bf16 value is exact, so both sums are exact for ordinary rows and
    // var = E[v^2] - mean^2 is within a few binary64 ulps of the two-pass
    // value unless |mean| dwarfs the spread by many orders of magnitude.
    double s1 = 0.0, s2 = 0.0;
#pragma unroll
    for (int k = 0; k < V; ++k) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const double d = (double)v[k][i];
            s1 += d;
            s2 = __builtin_fma(d, d, s2);
        }
    }
    s1 = wave_sum(s1);
    s2 = wave_sum(s2);
    if (WPR > 1) {
        if (lane == 0) {
            scratch[rw][sw][0] = s1;
            scratch[rw][sw][1] = s2;
        }
        __syncthreads();
        s1 = 0.0;
        s2 = 0.0;
#pragma unroll
        for (int w = 0; w < WPR; ++w) {
            s1 += scratch[rw][w][0];
            s2 += scratch[rw][w][1];
        }
    }
    if (!active) {
        if constexpr (kFp4) {  // rows [rows, round_up(rows, 128)) of the scale matrix are zero
            if (row < a.fp4_rows_padded) {
                const int groups = H >> 4;
                for (int gi = sw * 64 + lane; gi < groups; gi += 64 * WPR)
                    a.fp4_scales[fp4_scale_offset(row, gi, groups, a.fp4_tiled)] = 0;
            }
        }
        return;
    }
    // mean = s1 / hidden within an ulp of binary64 (reciprocal from the host),
    // factor = 1 / sqrt(var + eps) by binary64 Newton steps; both then rounded
    // once to fp32.
    const double mean = s1 * inv_hidden;
    const double var = __builtin_fmax(s2 * inv_hidden - mean * mean, 0.0);
    const float factor = rsqrt_rn32(var + (double)a.eps);
    const float mean32 = (float)mean;

    // 5. Modulate, quantise, store.
#pragma unroll
    for (int k = 0; k < V; ++k) {
        // The FP4 path keeps every lane to the end: the two lanes of a
        // 16-element group exchange their maxima (columns past the row end
        // come in whole pairs and only pair with each other).
        if (!kFp4 && !ok[k]) continue;
        const int c = 64 * (sw + WPR * k) + lane;
        float ops[8], sh[8];
        if (kHoist || kStage) {
            unpack8(kStage ? stage[(0 * V + k) * 64 + lane] : cin[0][k], ops);
            unpack8(kStage ? stage[(1 * V + k) * 64 + lane] : cin[1][k], sh);
#pragma unroll
            for (int i = 0; i < 8; ++i) ops[i] = 1.0f + ops[i];
        } else if (ok[k]) {
            col8<kLds>(cols, a, 0, c, ops);
            col8<kLds>(cols, a, 1, c, sh);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) ops[i] = sh[i] = 0.0f;
        }
        // m = norm * (1 + scale) + shift in fp32, from the bf16 norm.
        float m[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float norm = round_bf16((v[k][i] - mean32) * factor);
            m[i] = __builtin_fmaf(norm, ops[i], sh[i]);
        }
        // y = bf16(m): packed for the store, and as fp32 values (each from one
        // conversion) when a quantised output is formed from it.
        if constexpr (kFp4) {
            float yv[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) yv[i] = round_bf16(m[i]);
            // 16-element group = this lane's 8 values and its neighbour's
            // (lanes 2g and 2g + 1 hold chunks 2g and 2g + 1 of the row).
            float amax = 0.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(yv[i]));
            const float other = __builtin_bit_cast(
                float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, amax), 0xB1, 0xF, 0xF, false));
            amax = __builtin_fmaxf(amax, other);  // quad_perm [1, 0, 3, 2]
            const float s_pre = div6_bf16(amax) * g4;  // amax is a bf16 value
            const uint32_t s8 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(
                                    __builtin_fminf(s_pre, 448.0f), 0.0f, 0, false) & 0xFFu;
            uint32_t packed = 0;
            if (s8 != 0) {
                const float kq = kLds ? kq_tab[s8] : g4 / e4m3_value_pos(s8);  // IEEE division
                float t[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) t[i] = yv[i] * kq;
                packed = pack_e2m1x8(t);
            }
            if (ok[k]) {
                if (want_y)
                    store16(a.y + base + 8 * c,
                            (u32x4){pack_bf16_exact(yv[0], yv[1]), pack_bf16_exact(yv[2], yv[3]),
                                    pack_bf16_exact(yv[4], yv[5]), pack_bf16_exact(yv[6], yv[7])});
                store4(a.fp4 + row * (H >> 1) + 4 * c, packed);
                if ((lane & 1) == 0)
                    a.fp4_scales[fp4_scale_offset(row, c >> 1, H >> 4, a.fp4_tiled)] = (uint8_t)s8;
            }
        } else if (want_q) {  // q from the bf16 y, stored or not
            float yv[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) yv[i] = round_bf16(m[i]);
            if (want_y)
                store16(a.y + base + 8 * c,
                        (u32x4){pack_bf16_exact(yv[0], yv[1]), pack_bf16_exact(yv[2], yv[3]),
                                pack_bf16_exact(yv[4], yv[5]), pack_bf16_exact(yv[6], yv[7])});
            const uint32_t q0 = pack_e4m3x4(clamp_e4m3(yv[0] * inv), clamp_e4m3(yv[1] * inv),
                                            clamp_e4m3(yv[2] * inv), clamp_e4m3(yv[3] * inv));
            const uint32_t q1 = pack_e4m3x4(clamp_e4m3(yv[4] * inv), clamp_e4m3(yv[5] * inv),
                                            clamp_e4m3(yv[6] * inv), clamp_e4m3(yv[7] * inv));
            store8(a.q + base + 8 * c, (u32x2){q0, q1});
        } else {  // y only
            store16(a.y + base + 8 * c, (u32x4){pack_bf16(m[0], m[1]), pack_bf16(m[2], m[3]),
                                                pack_bf16(m[4], m[5]), pack_bf16(m[6], m[7])});
        }
    }
}

template <int MODE, int WPR, int RPW, int V, bool kLds, bool kFp4, bool kExact, bool kHoist,
          bool kStage, bool kDual>
hipError_t launch_kernel(const NormModulateArgs& a0, const NormModulateArgs& a1, int64_t blocks0,
                         uint64_t blocks, hipStream_t stream) {
    const int H = a0.hidden;
    const size_t lds = kLds ? ((size_t)kColVecs<MODE> * H + (kFp4 ? 128 : 0)) * sizeof(float)
                            : (kStage ? (size_t)WPR * 2 * V * 64 * sizeof(u32x4) : 0);
    hipLaunchKernelGGL(
        (norm_modulate_fp8_kernel<MODE, WPR, RPW, V, kLds, kFp4, kExact, kHoist, kStage, kDual>),
        dim3((unsigned)blocks), dim3(64 * WPR * RPW), lds, stream, a0, a1, blocks0, 1.0 / (double)H);
    return hipGetLastError();
}

// Launch with WPR waves per row, RPW rows per workgroup and V chunks per lane
// (V * 64 * WPR >= hidden / 8); kLds stages the column vectors in LDS as fp32,
// kStage (exact fits only) parks them raw in LDS for every row slot. a1 is the
// second row set (a1.rows == 0: none); both share a0's width.
template <int MODE, int WPR, int RPW, int V, bool kLds, bool kFp4, bool kHoist = false,
          bool kStage = false>
hipError_t launch_geom(const NormModulateArgs& a0, const NormModulateArgs& a1, hipStream_t stream) {
    const int64_t rows0 = kFp4 ? a0.fp4_rows_padded : a0.rows;
    const int64_t rows1 = kFp4 ? a1.fp4_rows_padded : a1.rows;
    const int64_t blocks0 = (rows0 + RPW - 1) / RPW;
    const uint64_t blocks = (uint64_t)(blocks0 + (rows1 + RPW - 1) / RPW);
    if (blocks * (64 * WPR * RPW) >= kMaxGridLanes) return kGridTooLarge;
    const int H = a0.hidden;
    if (kStage && H != 512 * WPR * V) return hipErrorInvalidValue;  // chosen for exact fits only
    const bool exact = kStage || (MODE == kPlain && H == 512 * WPR * V);
    if constexpr (MODE == kPlain && !kFp4) {
        if (rows1 > 0)
            return exact ? launch_kernel<MODE, WPR, RPW, V, kLds, kFp4, true, kHoist, kStage, true>(
                               a0, a1, blocks0, blocks, stream)
                         : launch_kernel<MODE, WPR, RPW, V, kLds, kFp4, false, kHoist, false, true>(
                               a0, a1, blocks0, blocks, stream);
    }
    return exact ? launch_kernel<MODE, WPR, RPW, V, kLds, kFp4, true, kHoist, kStage, false>(
                       a0, a1, blocks0, blocks, stream)
                 : launch_kernel<MODE, WPR, RPW, V, kLds, kFp4, false, kHoist, false, false>(
                       a0, a1, blocks0, blocks, stream);
}

// Geometries measured on MI355X (time per call over back-to-back launches
// with rotating buffers), at hidden 3072 unless stated:
//  - fewer than 1024 rows (latency-bound): six waves per row, one row per
//    workgroup, column vectors loaded from L2 together with the row
//    (127 rows: 3.7 -> 3.3 us, against 2.4 us for an empty kernel);
//  - plain variant, many rows: two waves per row, four rows per workgroup;
//    at hidden 6144 (FLUX.2) six waves per row and two rows per workgroup
//    with both outputs; with the FP8 output only, four waves per row and two
//    rows per workgroup with scale and shift parked in LDS (kStage) --
//    20.1 -> 19.3 us at 4608 x 6144, against one row per workgroup reading
//    them from L2 after the statistics;
//  - residual variants, many rows: one wave per row, eight rows per workgroup,
//    column vectors staged in LDS when they fit in 48 KiB.
template <int MODE, bool kFp4>
hipError_t launch_mode(const NormModulateArgs& a, const NormModulateArgs& a1, hipStream_t stream) {
    const int cpr = a.hidden / 8;
    if (a.rows + a1.rows < 1024) {
        switch ((cpr + 383) / 384) {
            case 1: return launch_geom<MODE, 6, 1, 1, false, kFp4, true>(a, a1, stream);
            case 2: return launch_geom<MODE, 6, 1, 2, false, kFp4, true>(a, a1, stream);
            default: return launch_geom<MODE, 6, 1, 3, false, kFp4, true>(a, a1, stream);  // up to 1152 chunks
        }
    }
    if constexpr (MODE == kPlain && !kFp4) {
        // Two waves per row and four rows per workgroup hold 16 rows per CU at
        // once (53 VGPRs, 8 waves per SIMD), 4096 rows on the 256 CUs; a
        // launch with up to 6144 rows (Qwen-Image's 4096 image + 512 text
        // rows) fits in one resident round with one wave per row instead (76
        // VGPRs, 24 rows per CU): 12.9 against 15.3 us at 4608 x 3072, where
        // a second round of workgroups would wait for the first.
        const int64_t rows = a.rows + a1.rows;
        if (rows > 4096 && rows <= 6144 && cpr > 320 && cpr <= 384)
            return launch_geom<MODE, 1, 1, 6, false, kFp4>(a, a1, stream);
    }
    if constexpr (MODE == kPlain) {
        if (cpr > 384 && cpr <= 768) {
            if (a.y) return launch_geom<MODE, 6, 2, 2, false, kFp4>(a, a1, stream);
            if constexpr (!kFp4) {
                if (a.hidden == 512 * 4 * 3) return launch_geom<MODE, 4, 2, 3, false, kFp4, false, true>(a, a1, stream);
            }
            return launch_geom<MODE, 4, 1, 3, false, kFp4>(a, a1, stream);
        }
    }
    if constexpr (MODE != kPlain) {
        if (cpr > 384) goto two_waves;
        const bool lds = (size_t)kColVecs<MODE> * a.hidden * sizeof(float) <= kLdsColsMax;
        switch ((cpr + 63) / 64) {
#define DIT_NM_ONE_WAVE(VV)                                                                    \
    case VV:                                                                                   \
        return lds ? launch_geom<MODE, 1, 8, VV, true, kFp4>(a, a1, stream)                             \
                   : launch_geom<MODE, 1, 8, VV, false, kFp4>(a, a1, stream);
            DIT_NM_ONE_WAVE(1) DIT_NM_ONE_WAVE(2) DIT_NM_ONE_WAVE(3)
            DIT_NM_ONE_WAVE(4) DIT_NM_ONE_WAVE(5) DIT_NM_ONE_WAVE(6)
#undef DIT_NM_ONE_WAVE
        }
    }
two_waves:
    switch ((cpr + 127) / 128) {
        case 1: return launch_geom<MODE, 2, 4, 1, false, kFp4>(a, a1, stream);
        case 2: return launch_geom<MODE, 2, 4, 2, false, kFp4>(a, a1, stream);
        case 3: return launch_geom<MODE, 2, 4, 3, false, kFp4>(a, a1, stream);
        case 4: return launch_geom<MODE, 2, 4, 4, false, kFp4>(a, a1, stream);
        case 5: case 6: return launch_geom<MODE, 2, 4, 6, false, kFp4>(a, a1, stream);
        default: return launch_geom<MODE, 2, 4, 8, false, kFp4>(a, a1, stream);  // up to 1024 chunks
    }
}

template <bool kFp4>
hipError_t launch_modes(const NormModulateArgs& a, const NormModulateArgs& a1, hipStream_t stream) {
    if (a.residual == nullptr) return launch_mode<kPlain, kFp4>(a, a1, stream);
    if (a.bias == nullptr) return launch_mode<kResidual, kFp4>(a, a1, stream);
    return launch_mode<kBiasResidual, kFp4>(a, a1, stream);
}

}  // namespace

hipError_t launch_norm_modulate_fp8(const NormModulateArgs& a, hipStream_t stream) {
    NormModulateArgs none = a;  // no second row set
    none.rows = 0;
    none.fp4_rows_padded = 0;
    return a.fp4 ? launch_modes<true>(a, none, stream) : launch_modes<false>(a, none, stream);
}

// The geometry is chosen as for a0 with the two row counts added; a set with
// no rows is left out.
hipError_t launch_norm_modulate_fp8_dual(const NormModulateArgs& a0, const NormModulateArgs& a1,
                                         hipStream_t stream) {
    if (a0.rows == 0) return launch_norm_modulate_fp8(a1, stream);
    if (a1.rows == 0) return launch_norm_modulate_fp8(a0, stream);
    return launch_mode<kPlain, false>(a0, a1, stream);
}

}  // namespace dit

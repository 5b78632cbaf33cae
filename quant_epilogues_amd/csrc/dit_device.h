// dit_device.h -- device-side helpers shared by the gfx950 epilogue kernels:
// bf16 / FP8 / FP4 conversions, the exactly-rounded sums the epilogues need,
// and wave64 reductions.
//
// Conversions use the gfx950 conversion instructions (round to nearest even;
// sign kept on zero):
//   v_cvt_pk_bf16_f32          fp32 -> bf16
//   v_cvt_pk_fp8_f32           fp32 in [-448, 448] -> OCP E4M3FN
//   v_cvt_scalef32_pk_fp4_f32  fp32 -> E2M1 with unit scale (saturates at 6;
//                              first source in the low nibble)
// The helpers below that wrap them (pack_bf16, round_bf16, clamp_e4m3 +
// pack_e4m3x4, pack_e2m1x8) are checked on the GPU against encoders written
// from the format definitions: on every fp32 value whose upper 16 bits are
// any finite pattern and whose lower 16 bits lie within 2 ulps of 0 or of
// 0x8000 -- every bf16 value, every bf16 rounding midpoint, and every E4M3
// and E2M1 rounding boundary with its neighbours, since those boundaries have
// few significant bits -- plus 2^22 random fp32 values.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dit {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // 16 bytes: 8 bf16
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));  // 8 bytes

// Cached loads: row-broadcast vectors (scale, shift, gate, bias, weights,
// cos/sin) that many workgroups re-read from L2.
__device__ __forceinline__ u32x4 load16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
// Streaming loads and stores: tensors touched exactly once. The non-temporal
// hint keeps them from displacing the broadcast vectors in L2 and measurably
// raises sustained HBM bandwidth on gfx950.
__device__ __forceinline__ u32x4 stream_load16(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void store16(void* p, u32x4 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}
__device__ __forceinline__ void store8(void* p, u32x2 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x2*>(p));
}
__device__ __forceinline__ void store4(void* p, uint32_t v) {
    __builtin_nontemporal_store(v, reinterpret_cast<uint32_t*>(p));
}

// ---- bf16 ------------------------------------------------------------------

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two fp32 -> two bf16 (round to nearest even), a in the low half.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

// bf16(v) (round to nearest even) as the fp32 value it denotes, in one
// conversion: packing (0, v) leaves bf16(v) in the high half over a zero low
// half, which is exactly the fp32 bit pattern of that bf16 value.
__device__ __forceinline__ float round_bf16(float v) { return __uint_as_float(pack_bf16(0.0f, v)); }

// Two fp32 values that are already bf16 values -> one word of two bf16 (a in
// the low half): their high halves, gathered with one byte permute.
__device__ __forceinline__ uint32_t pack_bf16_exact(float a, float b) {
    return __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u);
}

// 8 bf16 held in 16 bytes <-> 8 floats.
__device__ __forceinline__ void unpack8(const u32x4& v, float (&f)[8]) {
    f[0] = bf_lo(v.x); f[1] = bf_hi(v.x);
    f[2] = bf_lo(v.y); f[3] = bf_hi(v.y);
    f[4] = bf_lo(v.z); f[5] = bf_hi(v.z);
    f[6] = bf_lo(v.w); f[7] = bf_hi(v.w);
}
__device__ __forceinline__ u32x4 pack8(const float (&f)[8]) {
    return (u32x4){pack_bf16(f[0], f[1]), pack_bf16(f[2], f[3]),
                   pack_bf16(f[4], f[5]), pack_bf16(f[6], f[7])};
}

// bf16 of the EXACT sums p[i] + r[i] of fp32 values (one rounding each), two
// per word, element 2j in the low half of word j. The callers' p is a product
// of two bf16 values, exact in fp32 (8 x 8 significant bits) for |p| below
// 2^128, the bound of the library's input domain; a product too small for
// fp32 keeps only its sign, which can turn a -0 result into +0. Checking for
// both in the kernel measured 2-7% slower, so they stay outside the domain.
// The fp32 sum s = RN32(p + r)
// already rounds correctly to bf16 unless s lands exactly on a bf16 midpoint
// (rounding is monotone and bf16 midpoints are fp32 values) AND the fp32 sum
// was inexact; then the TwoSum error term says on which side the exact sum
// lies. For a bf16 product p and a bf16 r the fp32 sum is usually exact, and
// exact sums sit on bf16 midpoints often (~1/256), so the test is two-level,
// each level a wave-uniform branch: any midpoint (common), then any inexact
// midpoint (rare). The sum is inexact iff s - p != r or s - r != p (whichever
// operand is larger in magnitude, its difference with s is exact).
__device__ __forceinline__ void pack8_exact_sum(const float (&p)[8], const float (&r)[8],
                                                uint32_t (&w)[4]) {
    float s[8];
    bool mid = false;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        s[i] = p[i] + r[i];
        mid |= (__float_as_uint(s[i]) & 0xFFFFu) == 0x8000u;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = pack_bf16(s[2 * j], s[2 * j + 1]);
    if (__builtin_amdgcn_ballot_w64(mid) == 0) return;
    uint32_t fix = 0;  // bitwise, branch-free: computed for all 8 values
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t m = (__float_as_uint(s[i]) & 0xFFFFu) == 0x8000u;
        const uint32_t inexact = ((s[i] - p[i]) != r[i]) | ((s[i] - r[i]) != p[i]);
        fix |= m & inexact;
    }
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(fix != 0) == 0, 1)) return;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t u = __float_as_uint(s[i]);
        if ((u & 0xFFFFu) != 0x8000u) continue;
        const float bv = s[i] - p[i];
        const float e = (p[i] - (s[i] - bv)) + (r[i] - bv);
        if (e == 0.0f) continue;  // an exact tie: the even choice stands
        const uint32_t h = (u >> 16) + (((e > 0.0f) == (s[i] > 0.0f)) ? 1u : 0u);
        const int sh = (i & 1) * 16;
        w[i / 2] = (w[i / 2] & ~(0xFFFFu << sh)) | (h << sh);
    }
}

// ---- FP8 E4M3FN ------------------------------------------------------------

__device__ __forceinline__ float clamp_e4m3(float v) {
    return __builtin_amdgcn_fmed3f(v, -448.0f, 448.0f);
}

// Four values already clamped to [-448, 448] -> four E4M3 bytes (a lowest).
// The first conversion writes the low half and keeps the high half of its
// third operand, which the second conversion then overwrites: any register
// will do there, so `a`'s own bits are passed instead of a zeroed one.
__device__ __forceinline__ uint32_t pack_e4m3x4(float a, float b, float c, float d) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __float_as_int(a), false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}

// a / 6 (IEEE fp32, round to nearest even) for a non-negative bf16 value a
// held in fp32: the product with RN(1/6) and one FMA correction step. It
// equals the IEEE quotient for every non-negative finite bf16 value (with
// fp32 denormals preserved, as these kernels run), checked exhaustively on
// the GPU and, compiled for the host, on the CPU; +inf passes through.
__host__ __device__ __forceinline__ float div6_bf16(float a) {
    const float c = 0x1.555556p-3f;  // RN(1/6)
    const float q0 = a * c;
    const float q = __builtin_fmaf(__builtin_fmaf(-q0, 6.0f, a), c, q0);
    return a == __builtin_inff() ? a : q;
}

// Value of a non-negative E4M3FN code (sign bit clear, not NaN).
__device__ __forceinline__ float e4m3_value_pos(uint32_t c) {
    const uint32_t e = c >> 3, m = c & 7u;
    return e ? __builtin_ldexpf((float)(8u + m), (int)e - 10)
             : __builtin_ldexpf((float)m, -9);
}

// ---- FP4 E2M1 ----------------------------------------------------------------

// Eight values -> eight E2M1 nibbles in one dword (element 0 in the low nibble).
__device__ __forceinline__ uint32_t pack_e2m1x8(const float (&t)[8]) {
    uint32_t w = 0;
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, t[0], t[1], 1.0f, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, t[2], t[3], 1.0f, 1);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, t[4], t[5], 1.0f, 2);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, t[6], t[7], 1.0f, 3);
    return w;
}

// Byte offset of scale (m, k) of an FP4 group-scale matrix with `groups`
// scales per row: row-major, or 128-row x 4-column tiles of 512 bytes (tile
// column fastest) with rows interleaved as (m % 32, (m / 32) % 4) inside.
__device__ __forceinline__ int64_t fp4_scale_offset(int64_t m, int k, int groups, bool tiled) {
    if (!tiled) return m * groups + k;
    return ((m >> 7) * (groups >> 2) + (k >> 2)) * 512 + (m & 31) * 16 + ((m >> 5) & 3) * 4 + (k & 3);
}

// ---- reciprocal square root -------------------------------------------------

// RN32(1 / sqrt(v)) for any v >= 0 held in binary64 (row statistics of bf16
// data reach far beyond the fp32 range: a row holding 1e30 has a variance
// near 1e57). v is first scaled by an even power of two into [0.5, 2) --
// exact in binary64 -- so that the fp32 reciprocal-sqrt seed neither
// overflows nor underflows; two Newton steps in binary64 (error a few
// binary64 ulps) follow, the scaling is undone exactly, and the result is
// rounded once to fp32. It differs from the correctly rounded value only when
// 1/sqrt(v) lies within a few binary64 ulps of an fp32 rounding boundary.
__device__ __forceinline__ float rsqrt_rn32(double v) {
    if (v == 0.0) return __builtin_inff();
    if (v == __builtin_inf()) return 0.0f;
    int e;
    double m = __builtin_frexp(v, &e);  // v = m * 2^e, m in [0.5, 1)
    if (e & 1) {                        // make the exponent even: m in [1, 2)
        m *= 2.0;
        e -= 1;
    }
    double y = (double)__builtin_amdgcn_rsqf((float)m);
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const double t = m * y;
        const double err = __builtin_fma(-t, y, 1.0);  // 1 - m y^2
        y = __builtin_fma(0.5 * y, err, y);
    }
    return (float)__builtin_ldexp(y, -(e / 2));  // 1/sqrt(v) = y * 2^(-e/2)
}

// ---- wave64 reductions --------------------------------------------------------

// DPP move of a 64-bit value (both halves with the same lane pattern). The
// patterns used here (quad permutes, row mirrors) read a lane of the same
// 16-lane row for every lane, and all rows and banks are enabled, so every
// lane is written and no prior destination value is needed.
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const int lo = __builtin_amdgcn_mov_dpp((int)(uint32_t)u, CTRL, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_mov_dpp((int)(uint32_t)(u >> 32), CTRL, 0xF, 0xF, false);
    return __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint64_t)(uint32_t)lo);
}

// Sum over each 16-lane row; every lane of the row gets the same bits.
// quad_perm [1,0,3,2] and [2,3,0,1] sum a quad, row_half_mirror pairs the two
// quads of each 8 lanes, row_mirror the two halves of the row.
__device__ __forceinline__ double row16_sum(double v) {
    v += dpp_f64<0xB1>(v);
    v += dpp_f64<0x4E>(v);
    v += dpp_f64<0x141>(v);
    v += dpp_f64<0x140>(v);
    return v;
}

// Sum over the whole wave64; every lane gets the same bits.
__device__ __forceinline__ double wave_sum(double v) {
    v = row16_sum(v);
    v += __shfl_xor(v, 16, 64);
    v += __shfl_xor(v, 32, 64);
    return v;
}

// Sums of two binary64 values per thread over the whole workgroup (blockDim.x
// a multiple of 64, at most 1024). Every thread receives the same bits: waves
// reduce with wave_sum, then each thread adds the per-wave partials in wave
// order. `scratch` holds 32 doubles of LDS; the call contains __syncthreads.
__device__ __forceinline__ void block_sum2(double& a, double& b, double* scratch) {
    a = wave_sum(a);
    b = wave_sum(b);
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        scratch[wave] = a;
        scratch[16 + wave] = b;
    }
    __syncthreads();
    const int nwaves = blockDim.x >> 6;
    a = 0.0;
    b = 0.0;
    for (int w = 0; w < nwaves; ++w) {
        a += scratch[w];
        b += scratch[16 + w];
    }
}

}  // namespace dit

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
// Layout on gfx950: one workgroup per (row, tile of chunks), numbered in
// address order. FP8: a workgroup is one wave and each lane takes one
// 8-element chunk (one 16-byte streaming load -> one 8-byte store), so every
// load instruction of a wave reads 1 KiB contiguously. FP4: a workgroup is
// one wave and each lane takes one 16-byte half of a 16-element group per
// load (the two halves of a group sit in adjacent lanes and exchange their
// maxima), so FP4 loads are contiguous 1 KiB per instruction too. Chunks and
// groups never straddle the branch boundary because both widths are
// multiples of 16.
#include "dit_device.h"
#include "kernels.h"

namespace dit {
namespace {

// Lanes per workgroup: one wave. On MI355X one-wave workgroups streamed the
// FLUX.2 shape 6% faster than four-wave ones (they are dispatched and retired
// independently).
constexpr int kFp8Tile = 64;

__device__ __forceinline__ const uint16_t* cat_source(const TokenCatArgs& a, int64_t row, int c16) {
    const int a_chunks = (int)(a.a_cols >> 4);
    return c16 < a_chunks ? a.a + row * a.a_cols + 16 * c16
                          : a.b + row * a.b_cols + 16 * (c16 - a_chunks);
}

// The grid is (tile, row - row0): the tile index varies fastest, so consecutive
// workgroups sweep memory in address order. On MI355X this measured 5-10%
// faster than a grid whose fastest index is the row.
__device__ __forceinline__ void row_tile(int64_t row0, int64_t& row, int& tile) {
    row = row0 + blockIdx.y;
    tile = (int)blockIdx.x;
}

// FP8: U chunks of 8 elements per thread, kFp8Tile apart, so a workgroup
// covers U * kFp8Tile chunks and each load instruction of a wave reads 1 KiB
// of one row contiguously (one 16-byte streaming load -> one 8-byte store per
// chunk).
template <int U>
__global__ __launch_bounds__(kFp8Tile) void token_cat_fp8_kernel(TokenCatArgs a, int64_t row0) {
    int64_t row;
    int tile;
    row_tile(row0, row, tile);
    const int64_t cols = a.a_cols + a.b_cols;
    const int cpr = (int)(cols >> 3);
    const int a_chunks = (int)(a.a_cols >> 3);
    const float inv = 1.0f / *a.scale;  // IEEE division
    float f[U][8];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int c = (tile * U + u) * kFp8Tile + threadIdx.x;
        if (c >= cpr) continue;
        const uint16_t* src = c < a_chunks ? a.a + row * a.a_cols + 8 * c
                                           : a.b + row * a.b_cols + 8 * (c - a_chunks);
        unpack8(stream_load16(src), f[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int c = (tile * U + u) * kFp8Tile + threadIdx.x;
        if (c >= cpr) continue;
        const uint32_t w0 = pack_e4m3x4(clamp_e4m3(f[u][0] * inv), clamp_e4m3(f[u][1] * inv),
                                        clamp_e4m3(f[u][2] * inv), clamp_e4m3(f[u][3] * inv));
        const uint32_t w1 = pack_e4m3x4(clamp_e4m3(f[u][4] * inv), clamp_e4m3(f[u][5] * inv),
                                        clamp_e4m3(f[u][6] * inv), clamp_e4m3(f[u][7] * inv));
        store8(a.out + row * cols + 8 * c, (u32x2){w0, w1});
    }
}

// FP4, row-major scales: one wave per (row, 32 * kFp4Loads groups). Load t
// of lane l reads half-group piece 64 t + l of the wave's span (a 16-byte
// streaming load, element pieces in address order); the two halves of a
// group sit in adjacent lanes and exchange their maxima by DPP, so each lane
// quantises its 8 values (4 packed bytes) with the group's scale and even
// lanes write the scale byte. Rows past `rows` (up to the 128-row padding)
// only write zero scales. Two loads per lane measured best on MI355X at
// 4608 x 24576: 46.0 us, against 49.5 us for one lane per whole group in
// four-wave workgroups and 51.4 / 48.4 us for one / four loads per lane.
constexpr int kFp4Loads = 2;

__global__ __launch_bounds__(64) void token_cat_fp4_kernel(TokenCatArgs a, int64_t row0) {
    int64_t row;  // < round_up(rows, 128)
    int tile;
    row_tile(row0, row, tile);
    const int lane = threadIdx.x;
    const int64_t cols = a.a_cols + a.b_cols;
    const int groups = (int)(cols >> 4);
    const int p0 = tile * (64 * kFp4Loads);  // first half-group piece of the wave
    const float gscale = *a.scale;           // global inverse scale
    const bool live = row < a.rows;          // wave-uniform
    u32x4 raw[kFp4Loads];
#pragma unroll
    for (int t = 0; t < kFp4Loads; ++t) {
        const int pc = p0 + 64 * t + lane;
        const int g = pc >> 1;
        raw[t] = (live && g < groups) ? stream_load16(cat_source(a, row, g) + 8 * (pc & 1))
                                      : (u32x4){0, 0, 0, 0};
    }
#pragma unroll
    for (int t = 0; t < kFp4Loads; ++t) {
        const int pc = p0 + 64 * t + lane;
        const int g = pc >> 1;
        float f[8];
        unpack8(raw[t], f);
        float amax = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) amax = __builtin_fmaxf(amax, __builtin_fabsf(f[e]));
        const float other = __builtin_bit_cast(
            float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, amax), 0xB1, 0xF, 0xF, false));
        amax = __builtin_fmaxf(amax, other);  // quad_perm [1, 0, 3, 2]: the group's other half
        const float s_pre = div6_bf16(amax) * gscale;  // amax is a bf16 value
        const uint32_t s8 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(__builtin_fminf(s_pre, 448.0f),
                                                                      0.0f, 0, false) & 0xFFu;
        uint32_t w = 0;
        if (s8 != 0) {
            const float kq = gscale / e4m3_value_pos(s8);  // IEEE division
            float q[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) q[e] = f[e] * kq;
            w = pack_e2m1x8(q);
        }
        if (g < groups) {
            if (live) store4(a.out + row * (cols >> 1) + 4 * pc, w);
            if ((lane & 1) == 0) a.out_scales[row * groups + g] = (uint8_t)s8;
        }
    }
}

// FP4 with the scales in 128x4 tiles. Inside a tile, the 32 rows m with the
// same m % 32 / 8 hold one contiguous 128-byte line per tile column (4
// groups): rows m0 + 32 i + r (i < 4, r < 8) for m0 = 128 t + 8 j, and dword
// 4 r + i of the line holds the scales of row m0 + 32 i + r. A workgroup
// takes such a 32-row set over kTiledCols tile columns (kTiledGroups groups,
// 512 bytes of each row) with kTiledSetWaves waves. Set row s = 8 i + r is
// row m0 + 32 i + r. Each lane loads one 16-byte half group per row: a load
// instruction covers kTiledRowsPerLoad rows, 512 contiguous bytes each, and
// each wave issues its kTiledLoads loads (its four set rows) before
// quantising any. The two halves of a group sit in adjacent lanes and
// exchange their maxima by DPP. The scale bytes go to LDS, and after one
// barrier the first 128 lanes write every line whole, one dword per lane.
// Rows past `rows` (up to the 128-row padding) only contribute zero scales.
// Needs groups % 4 == 0 (whole tile columns). Measured on MI355X at
// 4608 x 24576 with 1, 2, 4, 8 and 16 waves per set: 50.5, 48.5, 46.7, 44.8
// and 62.8 us; eight tile columns with eight waves: 47.6 us.
constexpr int kTiledCols = 4;
constexpr int kTiledGroups = 4 * kTiledCols;                 // groups per workgroup
constexpr int kTiledLanesPerRow = 2 * kTiledGroups;         // one 16-byte half group per lane
constexpr int kTiledRowsPerLoad = 64 / kTiledLanesPerRow;   // rows per load instruction
constexpr int kTiledSetWaves = 8;                           // waves sharing a 32-row set
constexpr int kTiledLoads = 32 / kTiledRowsPerLoad / kTiledSetWaves;  // load instructions per wave

__global__ __launch_bounds__(64 * kTiledSetWaves) void token_cat_fp4_tiled_kernel(TokenCatArgs a) {
    __shared__ uint32_t sbuf32[32 * kTiledGroups / 4];  // [set row][group] scale bytes
    uint8_t* sbuf = reinterpret_cast<uint8_t*>(sbuf32);
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;  // this wave's rows: set rows 4 wv .. 4 wv + 3
    const int64_t cols = a.a_cols + a.b_cols;
    const int groups = (int)(cols >> 4);
    const int g0 = blockIdx.x * kTiledGroups;
    const int64_t m0 = (int64_t)(blockIdx.y >> 2) * 128 + (blockIdx.y & 3) * 8;
    const float gscale = *a.scale;  // global inverse scale
    const int piece = lane % kTiledLanesPerRow;
    const int gl = piece >> 1;  // group within the wave's span
    const int g = g0 + gl;
    const int half = piece & 1;
    u32x4 raw[kTiledLoads];
    bool ok[kTiledLoads];
#pragma unroll
    for (int t = 0; t < kTiledLoads; ++t) {
        const int sr = (wv * kTiledLoads + t) * kTiledRowsPerLoad + lane / kTiledLanesPerRow;
        const int64_t row = m0 + 32 * (sr >> 3) + (sr & 7);
        ok[t] = row < a.rows && g < groups;
        raw[t] = ok[t] ? stream_load16(cat_source(a, row, g) + 8 * half) : (u32x4){0, 0, 0, 0};
    }
#pragma unroll
    for (int t = 0; t < kTiledLoads; ++t) {
        const int sr = (wv * kTiledLoads + t) * kTiledRowsPerLoad + lane / kTiledLanesPerRow;
        const int64_t row = m0 + 32 * (sr >> 3) + (sr & 7);
        float f[8];
        unpack8(raw[t], f);
        float amax = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) amax = __builtin_fmaxf(amax, __builtin_fabsf(f[e]));
        const float other = __builtin_bit_cast(
            float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, amax), 0xB1, 0xF, 0xF, false));
        amax = __builtin_fmaxf(amax, other);  // quad_perm [1, 0, 3, 2]: the group's other half
        const float s_pre = div6_bf16(amax) * gscale;  // amax is a bf16 value
        const uint32_t s8 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(__builtin_fminf(s_pre, 448.0f),
                                                                      0.0f, 0, false) & 0xFFu;
        uint32_t w = 0;
        if (s8 != 0) {
            const float kq = gscale / e4m3_value_pos(s8);  // IEEE division
            float q[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) q[e] = f[e] * kq;
            w = pack_e2m1x8(q);
        }
        if (ok[t]) store4(a.out + row * (cols >> 1) + 8 * g + 4 * half, w);
        if (half == 0) sbuf[sr * kTiledGroups + gl] = (uint8_t)s8;
    }
    __syncthreads();
    // Dword d of the line of tile column kc holds the scales of groups
    // 4 kc .. 4 kc + 3 of set row 8 (d % 4) + d / 4.
    for (int idx = (int)threadIdx.x; idx < kTiledCols * 32; idx += 64 * kTiledSetWaves) {
        const int kc = idx >> 5, d = idx & 31;
        const int gc = g0 + 4 * kc;
        if (gc < groups) {
            const int sr = 8 * (d & 3) + (d >> 2);
            const uint32_t v = sbuf32[(sr * kTiledGroups + 4 * kc) >> 2];
            const int64_t line = ((m0 >> 7) * (groups >> 2) + (gc >> 2)) * 512 + (m0 & 31) * 16;
            store4(a.out_scales + line + 4 * d, v);
        }
    }
}

// One workgroup per (tile, row); rows go in launches of at most kRowsPerLaunch
// (the grid's y extent), usually one.
constexpr int64_t kRowsPerLaunch = 65536;

template <typename Kernel>
hipError_t launch_rows_tiles(Kernel kernel, int threads, const TokenCatArgs& a, int64_t rows,
                             int64_t per_tile, int64_t units_per_row, hipStream_t stream) {
    const int64_t tiles = (units_per_row + per_tile - 1) / per_tile;
    if ((uint64_t)tiles * threads >= kMaxGridLanes) return kGridTooLarge;
    for (int64_t row0 = 0; row0 < rows; row0 += kRowsPerLaunch) {
        const int64_t n = rows - row0 < kRowsPerLaunch ? rows - row0 : kRowsPerLaunch;
        hipLaunchKernelGGL(kernel, dim3((unsigned)tiles, (unsigned)n), dim3(threads), 0, stream, a,
                           row0);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

constexpr int kFp8ChunksPerThread = 1;

}  // namespace

// One 8-element chunk per thread in one-wave workgroups measured best on
// MI355X at 4608 x (6144 + 18432) (two chunks: 1% slower).
hipError_t launch_token_cat_fp8(const TokenCatArgs& a, hipStream_t stream) {
    return launch_rows_tiles(token_cat_fp8_kernel<kFp8ChunksPerThread>, kFp8Tile, a, a.rows,
                             (int64_t)kFp8ChunksPerThread * kFp8Tile, (a.a_cols + a.b_cols) / 8,
                             stream);
}

hipError_t launch_token_cat_fp4(const TokenCatArgs& a, hipStream_t stream) {
    const int64_t rows_padded = (a.rows + 127) / 128 * 128;
    if (a.scales_tiled) {
        const int64_t groups = (a.a_cols + a.b_cols) / 16;
        const int64_t chunks = (groups + kTiledGroups - 1) / kTiledGroups;
        for (int64_t set0 = 0; set0 < rows_padded / 32; set0 += kRowsPerLaunch) {
            const int64_t n = rows_padded / 32 - set0 < kRowsPerLaunch ? rows_padded / 32 - set0
                                                                       : kRowsPerLaunch;
            TokenCatArgs b = a;  // row sets [set0, set0 + n): shift the row origin
            b.a = a.a + set0 * 32 * a.a_cols;
            b.b = a.b ? a.b + set0 * 32 * a.b_cols : nullptr;
            b.out = a.out + set0 * 32 * ((a.a_cols + a.b_cols) / 2);
            b.out_scales = a.out_scales + set0 * 32 * groups;
            b.rows = a.rows - set0 * 32;
            hipLaunchKernelGGL(token_cat_fp4_tiled_kernel, dim3((unsigned)chunks, (unsigned)n),
                               dim3(64 * kTiledSetWaves), 0, stream, b);
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    return launch_rows_tiles(token_cat_fp4_kernel, 64, a, rows_padded, 32 * kFp4Loads,
                             (a.a_cols + a.b_cols) / 16, stream);
}

}  // namespace dit

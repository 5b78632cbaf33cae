// kernels.h -- argument blocks and launchers of the gfx950 epilogue kernels.
// Internal to libdit_epilogues: the C ABI (api.cpp) validates arguments on the
// host and then calls one launcher, which only enqueues work on the stream.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dit {

// A launch covers at most 2^32 lanes along its grid's x dimension. Launchers
// return kGridTooLarge, before calling HIP, for sizes that would need more.
constexpr uint64_t kMaxGridLanes = uint64_t(1) << 32;
constexpr hipError_t kGridTooLarge = hipErrorInvalidConfiguration;

// LayerNorm + AdaLN modulation + static FP8 or 16-element-group FP4
// (optionally after bias + gated residual). residual == nullptr selects the
// plain variant; fp4 != nullptr selects the FP4 output (q is then nullptr).
struct NormModulateArgs {
    uint16_t* y;             // [rows, hidden] bf16, or nullptr: not written
    uint8_t* q;              // [rows, hidden] e4m3, or nullptr: not computed
    uint16_t* r_out;         // [rows, hidden] bf16 (residual variant only)
    const uint16_t* x;       // [rows, hidden]
    const uint16_t* residual;  // [rows, hidden] or nullptr
    const uint16_t* bias;    // [hidden] or nullptr
    const uint16_t* gate;    // [hidden] (residual variant only)
    const uint16_t* scale;   // [hidden]
    const uint16_t* shift;   // [hidden]
    const float* input_scale;  // device scalar: FP8 scale (read only when q is written),
                               // or the FP4 global inverse scale
    uint8_t* fp4;              // [rows, hidden / 2] packed E2M1, or nullptr (then q / y only)
    uint8_t* fp4_scales;       // [fp4_rows_padded, hidden / 16] E4M3 group scales
    int64_t fp4_rows_padded;   // rows rounded up to a multiple of 128
    bool fp4_tiled;            // scales in 128x4 tiles (else row-major)
    int64_t rows;
    int32_t hidden;          // multiple of 8, <= kMaxHidden (one thread per 8 columns)
    float eps;
};
constexpr int kMaxHidden = 8192;
hipError_t launch_norm_modulate_fp8(const NormModulateArgs& a, hipStream_t stream);
// Two row sets of the plain LayerNorm + modulation + FP8 (no residual, no FP4)
// with the same hidden, in one launch: a0's rows, then a1's (either may have 0).
hipError_t launch_norm_modulate_fp8_dual(const NormModulateArgs& a0, const NormModulateArgs& a1,
                                         hipStream_t stream);

struct QkvArgs {
    uint16_t* joint[3];            // q, k, v outputs [txt + img, heads, 128]
    const uint16_t* img[3];        // strided views
    const uint16_t* txt[3];
    const uint16_t* img_w[2];      // q, k RMSNorm weights [128]
    const uint16_t* txt_w[2];
    const float* img_cos;
    const float* img_sin;
    const float* txt_cos;
    const float* txt_sin;
    int64_t rope_stride;           // elements between rows of the cos / sin tables
    int64_t img_rows, img_stride;  // stride in elements
    int64_t txt_rows, txt_stride;
    int32_t heads;
    float img_eps, txt_eps;
};
constexpr int kHeadDim = 128;
constexpr int kMaxHeads = 64;
constexpr int kQkvHeadsPerWave = 12;  // heads handled by one wave of the QKV kernel
hipError_t launch_qkv_epilogue(const QkvArgs& a, hipStream_t stream);

struct BiasMulAddArgs {
    uint16_t* y;
    const uint16_t* x;
    const uint16_t* bias;  // nullptr: no bias
    const uint16_t* gate;
    const uint16_t* residual;
    int64_t rows;
    int64_t hidden;        // multiple of 8
};
hipError_t launch_bias_mul_add(const BiasMulAddArgs& a, hipStream_t stream);

struct TokenCatArgs {
    uint8_t* out;
    uint8_t* out_scales;   // FP4 only
    bool scales_tiled;     // FP4: scales in 128x4 tiles (else row-major)
    const uint16_t* a;
    const uint16_t* b;
    int64_t a_cols, b_cols, rows;
    const float* scale;    // device scalar
};
hipError_t launch_token_cat_fp8(const TokenCatArgs& a, hipStream_t stream);
hipError_t launch_token_cat_fp4(const TokenCatArgs& a, hipStream_t stream);

}  // namespace dit

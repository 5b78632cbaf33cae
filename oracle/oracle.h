/*
 * oracle.h -- plain, slow CPU oracle for the fused DiT-block epilogues.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark may load this library. It shares no code,
 * header, table or helper with the GPU library, and the GPU library never
 * calls it.
 *
 * Every buffer here is HOST memory. BF16 tensors travel as their raw 16-bit
 * patterns (uint16_t), FP8 E4M3 and packed FP4 as bytes. All matrices are
 * row-major. The pre-rounding outputs (`*_pre`) are optional (may be NULL);
 * they hand the test's tolerance checker the exact value that was rounded.
 *
 * Sources (the pages these definitions are read from):
 *   [QKV]  sglang PR 37123 page (Qwen-Image FP8 QKV fusion + fused epilogue)
 *   [NSS]  sglang PR 37156 page (Qwen-Image norm + FP8 activation quant fusion)
 *   [FX2]  sglang PR 37162 page (FLUX.2 FP8 fusions, token-cat + FP8)
 *   [BIAS] sglang PR 37116 page (Qwen-Image output-bias absorption)
 *   [FP4]  sglang PR 37141 page (FLUX.2 token concatenation + NVFP4)
 */
#ifndef DIT_ORACLE_H
#define DIT_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- format codecs, written from the format definitions ---------------- */

/* Nearest bfloat16 to a binary32 / binary64 value, ties to even. */
uint16_t oracle_bf16_from_f32(float v);
uint16_t oracle_bf16_from_f64(double v);
/* Nearest bfloat16 to the EXACT real sum a + b (one rounding). */
uint16_t oracle_bf16_of_exact_sum(double a, double b);
float oracle_f32_from_bf16(uint16_t h);

/* OCP E4M3FN: nearest finite value, ties to even code, |v| > 448 -> 448. */
uint8_t oracle_e4m3_encode(float v);
double oracle_e4m3_decode(uint8_t code);
/* E2M1: nearest of {0, .5, 1, 1.5, 2, 3, 4, 6}, ties to even code, |v| > 6 -> 6. */
uint8_t oracle_e2m1_encode(float v);
double oracle_e2m1_decode(uint8_t code);

/* Bulk forms for the exhaustive codec tests. */
void oracle_bf16_from_f32_n(const float* in, uint16_t* out, int64_t n);
void oracle_bf16_from_f64_n(const double* in, uint16_t* out, int64_t n);
void oracle_bf16_of_exact_sum_n(const double* a, const double* b, uint16_t* out, int64_t n);
void oracle_e4m3_encode_n(const float* in, uint8_t* out, int64_t n);
void oracle_e2m1_encode_n(const float* in, uint8_t* out, int64_t n);

/* ---- row statistics ------------------------------------------------------ */

/* LayerNorm statistics of one bf16 row: mean32 = RN32(mean), factor32 =
 * RN32(1 / sqrt(var + eps)) with biased variance, both from binary64. */
void oracle_layernorm_stats(const uint16_t* v, int64_t n, float eps,
                            float* mean32, float* factor32);
/* RMSNorm inverse of one bf16 vector: RN32(1 / sqrt(mean(v^2) + eps)). */
float oracle_rms_inverse(const uint16_t* v, int64_t n, float eps);

/* ---- the five epilogues -------------------------------------------------- */

/* LayerNorm (no affine) + AdaLN scale/shift + static FP8 E4M3 quantisation.
 * y, q: [rows, hidden]; scale, shift: [hidden]. q_pre (optional): the clamped
 * fp32 value each FP8 code was rounded from. */
void oracle_norm_modulate_fp8(uint16_t* y, uint8_t* q, float* q_pre,
                              const uint16_t* x, const uint16_t* scale,
                              const uint16_t* shift, float input_scale,
                              int64_t rows, int64_t hidden, float eps);

/* Optional input bias + gated residual, then the same norm/modulate/FP8.
 * r_out = bf16(residual + gate * bf16(x + bias)) with one rounding; bias may
 * be NULL (no bias). */
void oracle_scale_residual_norm_modulate_fp8(
    uint16_t* r_out, uint16_t* y, uint8_t* q, float* q_pre,
    const uint16_t* x, const uint16_t* bias, const uint16_t* gate,
    const uint16_t* residual, const uint16_t* scale, const uint16_t* shift,
    float input_scale, int64_t rows, int64_t hidden, float eps);

/* Per-head RMSNorm of Q and K, interleaved RoPE, V copy, joint [text, image]
 * packing. Inputs are row-strided views (strides in elements); head h of a
 * row starts at element h * head_dim. cos/sin tables are [rows, head_dim/2]
 * per stream. Outputs joint_* are [txt_rows + img_rows, heads, head_dim]. */
void oracle_qkv_epilogue(
    uint16_t* joint_q, uint16_t* joint_k, uint16_t* joint_v,
    const uint16_t* img_q, const uint16_t* img_k, const uint16_t* img_v,
    int64_t img_rows, int64_t img_row_stride,
    const uint16_t* txt_q, const uint16_t* txt_k, const uint16_t* txt_v,
    int64_t txt_rows, int64_t txt_row_stride,
    const uint16_t* img_q_w, const uint16_t* img_k_w,
    const uint16_t* txt_q_w, const uint16_t* txt_k_w,
    const float* img_cos, const float* img_sin,
    const float* txt_cos, const float* txt_sin,
    int32_t heads, int32_t head_dim, float img_eps, float txt_eps);

/* y = bf16((bf16(x + bias)) * gate + residual) with one rounding of the
 * multiply-add; bias may be NULL (treated as zero). */
void oracle_bias_mul_add(uint16_t* y, const uint16_t* x, const uint16_t* bias,
                         const uint16_t* gate, const uint16_t* residual,
                         int64_t rows, int64_t hidden);

/* Static FP8 quantisation of the row concatenation [a | b]:
 * out [rows, a_cols + b_cols]. */
void oracle_token_cat_fp8(uint8_t* out, float* pre, const uint16_t* a,
                          int64_t a_cols, const uint16_t* b, int64_t b_cols,
                          int64_t rows, float input_scale);

/* 16-element-group FP4 (E2M1) quantisation of [a | b] with one E4M3 scale per
 * group. packed [rows, (a_cols+b_cols)/2] (low nibble = even element);
 * scales [round_up(rows,128), (a_cols+b_cols)/16] row-major, pad rows zero.
 * g is the global fp32 inverse scale. s_pre [rows, groups] and pre
 * [rows, cols] are optional. */
void oracle_token_cat_fp4(uint8_t* packed, uint8_t* scales, float* s_pre,
                          float* pre, const uint16_t* a, int64_t a_cols,
                          const uint16_t* b, int64_t b_cols, int64_t rows,
                          float g);

/* NVFP4 output on the LayerNorm path: y as oracle_norm_modulate_fp8, then
 * 16-element-group FP4 of the bf16 y (as oracle_token_cat_fp4). packed is
 * [rows, hidden/2], scales [round_up(rows, 128), hidden/16] (pad rows 0),
 * s_pre [rows, hidden/16] and pre [rows, hidden] optional. hidden % 16 == 0. */
void oracle_norm_modulate_fp4(uint16_t* y, uint8_t* packed, uint8_t* scales,
                              float* s_pre, float* pre, const uint16_t* x,
                              const uint16_t* scale, const uint16_t* shift,
                              float g, int64_t rows, int64_t hidden, float eps);
void oracle_scale_residual_norm_modulate_fp4(
    uint16_t* r_out, uint16_t* y, uint8_t* packed, uint8_t* scales, float* s_pre,
    float* pre, const uint16_t* x, const uint16_t* bias, const uint16_t* gate,
    const uint16_t* residual, const uint16_t* scale, const uint16_t* shift,
    float g, int64_t rows, int64_t hidden, float eps);

/* Rearranges a row-major FP4 scale matrix [rows_padded, groups] (rows_padded %
 * 128 == 0, groups % 4 == 0) into the 128x4 tile layout of FP4 GEMMs. */
void oracle_fp4_scales_to_128x4(uint8_t* out, const uint8_t* row_major,
                                int64_t rows_padded, int64_t groups);

#ifdef __cplusplus
}
#endif
#endif /* DIT_ORACLE_H */

/*
 * dit_epilogues.h -- C ABI of the fused, memory-bound, row-wise epilogues of a
 * diffusion-transformer block, implemented as HIP kernels for gfx950 (MI355X).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every tensor pointer is a DEVICE pointer. BF16 tensors are passed as
 *    void* (raw 16-bit bfloat16 patterns); FP8 E4M3FN and packed FP4 outputs
 *    as uint8_t*. Matrices are row-major; unless a stride argument says
 *    otherwise, rows are dense.
 *  - The caller owns and allocates every buffer. The library never allocates,
 *    frees or synchronises; each call enqueues its work on `stream` (a
 *    hipStream_t passed as void*; NULL is the default stream) and returns.
 *    Calls contain no host<->device copies and no host reads of device data,
 *    so they can be captured into a HIP graph.
 *  - Static quantisation scales (`input_scale_dev`, `scale_dev`) are device
 *    pointers to ONE fp32 value, read by the kernel only. Preconditions that
 *    are documented but NOT checked: scales are finite and > 0, inputs are
 *    finite, and no output overlaps any input or another output. Where a call
 *    forms gate * x before a once-rounded sum (dit_bias_mul_add and the gated
 *    residual of the dit_scale_residual_* calls), |gate * x| < 2^128 for
 *    every element: the product is formed in fp32, which is exact below that
 *    bound and overflows to +-inf above it. A product so small that fp32
 *    holds only its sign (|gate * x| < 2^-149) can give +0 where the exact
 *    sum is -0.
 *  - Return value: DIT_OK (0) or a dit_status code. On any refusal the call
 *    enqueues nothing and outputs are untouched, so a caller can fall back to
 *    an unfused path. The reason is also available from dit_last_error()
 *    (per thread). rows == 0 is a successful no-op.
 *  - Validation is host-only and happens before any HIP call: NULL pointers
 *    (DIT_ERR_NULL), negative or inconsistent sizes (DIT_ERR_SHAPE), pointers
 *    not 16-byte aligned (DIT_ERR_ALIGN), shapes outside the instantiated
 *    kernels or too large for one launch, whose grid may cover at most 2^32
 *    lanes (DIT_ERR_UNSUPPORTED). A failing launch returns DIT_ERR_HIP.
 *
 * Sources: the five sglang pull-request summary pages on prhub.com.cn that
 * describe these fusions (PRs 37123, 37156, 37162, 37116, 37141). Each entry
 * point names the page and section that define what it computes.
 */
#ifndef DIT_EPILOGUES_H
#define DIT_EPILOGUES_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DIT_ABI_VERSION 5

typedef enum dit_status {
    DIT_OK = 0,
    DIT_ERR_NULL = 1,        /* a required pointer is NULL                    */
    DIT_ERR_SHAPE = 2,       /* negative / inconsistent sizes or strides      */
    DIT_ERR_ALIGN = 3,       /* a pointer is not 16-byte aligned              */
    DIT_ERR_UNSUPPORTED = 4, /* valid arguments no kernel is built for        */
    DIT_ERR_HIP = 5          /* the HIP runtime refused the launch            */
} dit_status;

/* ABI version of the loaded library (DIT_ABI_VERSION at build time). */
int dit_abi_version(void);

/* Static, human-readable name of a status code (never NULL). */
const char* dit_status_string(int status);

/* Message describing the most recent refusal on the calling thread ("" if the
 * last call succeeded). The pointer stays valid until the thread's next call. */
const char* dit_last_error(void);

/*
 * LayerNorm without affine + AdaLN modulation + static FP8 E4M3 quantisation,
 * dual output.
 *
 * Defined by: sglang PR 37156 page ("Implementation breakdown" items 1-2 and
 * the norm_scale_shift excerpt under "Key source snippets"): one row per block;
 * LayerNorm without weight or bias with fp32 statistics; the normalised value
 * is rounded to bf16; y = bf16(norm * (1 + scale) + shift); the FP8 output is
 * e4m3(clamp(y * (1 / input_scale), -448, 448)). Both outputs are written.
 *
 *   y      [rows, hidden] bf16, out; NULLABLE: FP8-only output, the bf16 y is
 *          still formed (q is computed from it) but not written, as the FLUX.2
 *          variant on the sglang PR 37162 page ("Implementation breakdown"
 *          item 1) drops the bf16 intermediate
 *   q      [rows, hidden] E4M3FN bytes, out; NULLABLE: bf16-only output
 *          (input_scale_dev may then be NULL too). y and q are not both NULL.
 *   x      [rows, hidden] bf16, in
 *   scale, shift  [hidden] bf16, in (broadcast over rows)
 *   input_scale_dev  device fp32 scalar (static FP8 scale; q = y / scale)
 *   eps    LayerNorm epsilon (host fp32)
 *
 * Statistics: mean and biased variance per row; 1 / input_scale is IEEE fp32
 * division. hidden must be a multiple of 8 and at most 8192 (one workgroup
 * holds the row), else DIT_ERR_UNSUPPORTED.
 */
int dit_norm_modulate_fp8(void* y, uint8_t* q, const void* x, const void* scale,
                          const void* shift, const float* input_scale_dev,
                          int64_t rows, int64_t hidden, float eps, void* stream);

/*
 * dit_norm_modulate_fp8 for the two token streams of a double-stream DiT
 * block in ONE launch: the image rows and the text rows, each with its own
 * outputs, input, modulation vectors, FP8 input scale and epsilon, and one
 * shared hidden size. Each stream's results are exactly those of a
 * dit_norm_modulate_fp8 call on it alone.
 *
 * Defined by: sglang PR 37156 page (what each row computes, as
 * dit_norm_modulate_fp8); sglang PR 37123 page ("Implementation breakdown"
 * item 3: one fused kernel covers both the image and the text stream, each
 * with its own parameters, as dit_qkv_epilogue does). Qwen-Image's 512 text
 * rows alone leave most of the GPU idle for the launch; sharing the launch
 * with the 4096 image rows removes that launch's fixed cost.
 *
 *   img_y, img_q, img_x, img_scale, img_shift, img_input_scale_dev, img_eps:
 *       the image stream's arguments, as dit_norm_modulate_fp8 (y or q may be
 *       NULL, not both; [img_rows, hidden] and [hidden])
 *   txt_*   the same for the text stream
 *   img_rows, txt_rows  >= 0 each (a stream with 0 rows needs no pointers)
 *   hidden  shared; same limits as dit_norm_modulate_fp8 (a multiple of 8,
 *           at most 8192)
 */
int dit_norm_modulate_fp8_dual(void* img_y, uint8_t* img_q, const void* img_x,
                               const void* img_scale, const void* img_shift,
                               const float* img_input_scale_dev, int64_t img_rows, float img_eps,
                               void* txt_y, uint8_t* txt_q, const void* txt_x,
                               const void* txt_scale, const void* txt_shift,
                               const float* txt_input_scale_dev, int64_t txt_rows, float txt_eps,
                               int64_t hidden, void* stream);

/*
 * Optional input bias + gated residual, then the same LayerNorm + modulation +
 * FP8 as dit_norm_modulate_fp8, writing the new residual too.
 *
 * Defined by: sglang PR 37156 page ("Implementation breakdown" item 2: the
 * residual variant returns normalised + quantised + residual_out) and sglang
 * PR 37116 page ("Implementation breakdown" item 3: x + bias folded into the
 * gated-residual LayerNorm kernel; the fallback forms a bf16 x + bias first).
 *
 *   residual_out [rows, hidden] bf16, out:
 *       bf16(residual + gate * xb) with ONE rounding, xb = bf16(x + bias)
 *       (xb = x when bias is NULL); |gate * xb| below 2^128 (see the
 *       conventions above)
 *   y, q         as dit_norm_modulate_fp8 (either may be NULL), computed
 *                from residual_out; q == NULL is the bf16-only bias + gated
 *                residual norm of the sglang PR 37116 page
 *   x, residual  [rows, hidden] bf16, in
 *   bias         [hidden] bf16, in, NULLABLE
 *   gate, scale, shift  [hidden] bf16, in
 *   input_scale_dev, eps  as dit_norm_modulate_fp8
 *
 * Same shape limits as dit_norm_modulate_fp8.
 */
int dit_scale_residual_norm_modulate_fp8(void* residual_out, void* y, uint8_t* q,
                                         const void* x, const void* bias,
                                         const void* gate, const void* residual,
                                         const void* scale, const void* shift,
                                         const float* input_scale_dev,
                                         int64_t rows, int64_t hidden, float eps,
                                         void* stream);

/*
 * Layouts of the FP4 group-scale matrix of rows_padded = round_up(rows, 128)
 * rows and groups = columns / 16 scales per row:
 *   DIT_FP4_SCALES_ROW_MAJOR  scale (m, k) at byte m * groups + k
 *   DIT_FP4_SCALES_128X4      the tile layout FP4 GEMMs read, which the sglang
 *       PR 37141 page names (128x4, as FlashInfer) without spelling out; read
 *       as: 128-row x 4-column tiles of 512 bytes, tile (m / 128, k / 4) at
 *       byte ((m / 128) * (groups / 4) + k / 4) * 512, and inside it scale
 *       (m, k) at (m % 32) * 16 + ((m / 32) % 4) * 4 + k % 4. Needs groups % 4
 *       == 0 (columns a multiple of 64).
 * Either way the buffer holds rows_padded * groups bytes and the scales of
 * rows [rows, rows_padded) are 0x00.
 */
#define DIT_FP4_SCALES_ROW_MAJOR 0
#define DIT_FP4_SCALES_128X4 1

/*
 * LayerNorm + AdaLN modulation with NVFP4 output: the bf16 y of
 * dit_norm_modulate_fp8, quantised in 16-element groups exactly as the FP4
 * output of dit_token_cat_quant (E2M1 codes, one E4M3 scale per group from
 * the global inverse scale, row-major scales, zero scales on pad rows).
 *
 * Defined by: the Qwen-Image residual-norm + NVFP4 fusion that the sglang
 * PR 37123 and PR 37162 pages list among their related PRs (named only), read
 * as the composition of the LayerNorm path (sglang PR 37156 page) with the
 * group FP4 quantisation of the sglang PR 37141 page ("Implementation
 * breakdown" item 1).
 *
 *   y       [rows, hidden] bf16, out; NULLABLE (then only the FP4 output)
 *   packed  [rows, hidden / 2] bytes, out; element 2k in the low nibble
 *   scales  [round_up(rows, 128), hidden / 16] E4M3 bytes, out, in the layout
 *           scale_layout names; scales of pad rows are written as 0x00
 *   scale_layout  DIT_FP4_SCALES_ROW_MAJOR or DIT_FP4_SCALES_128X4 (then
 *           hidden must be a multiple of 64)
 *   x, scale, shift, eps  as dit_norm_modulate_fp8
 *   global_scale_dev  device fp32 scalar g: group scale e4m3(amax / 6 * g),
 *           element code e2m1(y * g / scale)
 *
 * hidden must be a multiple of 16 and at most 8192 (else DIT_ERR_UNSUPPORTED).
 * scales needs no alignment; the other tensors 16 bytes.
 */
int dit_norm_modulate_fp4(void* y, uint8_t* packed, uint8_t* scales, int32_t scale_layout,
                          const void* x, const void* scale, const void* shift,
                          const float* global_scale_dev, int64_t rows, int64_t hidden,
                          float eps, void* stream);

/*
 * Optional input bias + gated residual, then the same LayerNorm + modulation
 * with NVFP4 output (residual_out, y and FP4 as above and as
 * dit_scale_residual_norm_modulate_fp8).
 *
 * Defined by: the same related-PR fusion, composed with the gated residual
 * of the sglang PR 37156 and PR 37116 pages.
 */
int dit_scale_residual_norm_modulate_fp4(void* residual_out, void* y, uint8_t* packed,
                                         uint8_t* scales, int32_t scale_layout,
                                         const void* x, const void* bias,
                                         const void* gate, const void* residual,
                                         const void* scale, const void* shift,
                                         const float* global_scale_dev, int64_t rows,
                                         int64_t hidden, float eps, void* stream);

/*
 * QKV epilogue: per-head RMSNorm of Q and K, interleaved RoPE, V copy, and the
 * joint [text, image] packing, reading Q/K/V straight from the packed QKV GEMM
 * output through strided views.
 *
 * Defined by: sglang PR 37123 page ("Implementation breakdown" items 3-4 and
 * the forward excerpt under "Key source snippets"): Q and K get an RMS
 * normalisation per head with their stream's weight and epsilon, then
 * interleaved (non-NeoX) RoPE from an fp32 cache; V is copied; outputs are
 * written in [text, image] order.
 *
 *   joint_q, joint_k, joint_v  [txt_rows + img_rows, heads, head_dim] bf16, out;
 *       joint row j < txt_rows is text row j, row txt_rows + i is image row i
 *   img_q, img_k, img_v  bf16 in; row i, head h starts at element
 *       i * img_row_stride + h * head_dim (e.g. column views of a packed
 *       [img_rows, 3 * heads * head_dim] buffer, stride 3 * heads * head_dim)
 *   txt_q, txt_k, txt_v  the same for the text stream
 *   *_row_stride  in ELEMENTS; >= heads * head_dim and a multiple of 8
 *   img_q_w, img_k_w, txt_q_w, txt_k_w  [head_dim] bf16 RMSNorm weights
 *   img_cos, img_sin  fp32 tables with one row of head_dim / 2 entries per
 *       image row; txt_cos, txt_sin the same per text row. Pair (2i, 2i+1) of
 *       a row rotates by the angle whose cos/sin are entry i of that row:
 *       (a, b) -> (a cos - b sin, b cos + a sin)
 *   rope_row_stride  elements between consecutive rows of all four tables;
 *       >= head_dim / 2 and a multiple of 4. head_dim / 2 for dense tables;
 *       head_dim for one shared cache whose rows hold [cos | sin] (pass
 *       img_cos = cache + txt_rows * head_dim, img_sin = img_cos + head_dim / 2,
 *       txt_cos = cache, txt_sin = cache + head_dim / 2), as the FLUX.2 variant
 *       on the sglang PR 37162 page takes one cos/sin cache for both streams
 *   img_eps, txt_eps  RMSNorm epsilons
 *
 * head_dim must be 128 (else DIT_ERR_UNSUPPORTED); heads in [1, 64] (24 for
 * Qwen-Image, 48 for FLUX.2). Either stream may have zero rows.
 */
int dit_qkv_epilogue(void* joint_q, void* joint_k, void* joint_v,
                     const void* img_q, const void* img_k, const void* img_v,
                     int64_t img_rows, int64_t img_row_stride,
                     const void* txt_q, const void* txt_k, const void* txt_v,
                     int64_t txt_rows, int64_t txt_row_stride,
                     const void* img_q_w, const void* img_k_w,
                     const void* txt_q_w, const void* txt_k_w,
                     const float* img_cos, const float* img_sin,
                     const float* txt_cos, const float* txt_sin, int64_t rope_row_stride,
                     int32_t heads, int32_t head_dim, float img_eps, float txt_eps,
                     void* stream);

/*
 * Final gated residual with an absorbed output bias: y = (x + bias) * gate +
 * residual.
 *
 * Defined by: sglang PR 37116 page (the bias_mul_add excerpt under "Key source
 * snippets" and the review highlights): the bias add is rounded to bf16, then
 * the multiply-add is one native bf16 FMA, i.e. rounded ONCE.
 *
 *   y         [rows, hidden] bf16, out
 *   x, residual  [rows, hidden] bf16, in
 *   bias      [hidden] bf16, in, NULLABLE (no bias add)
 *   gate      [hidden] bf16, in
 *
 * hidden must be a multiple of 8 (and at most 2^30). |gate * (x + bias)| must
 * stay below 2^128 (see the conventions above).
 */
int dit_bias_mul_add(void* y, const void* x, const void* bias, const void* gate,
                     const void* residual, int64_t rows, int64_t hidden,
                     void* stream);

/* Quantisation kinds of dit_token_cat_quant. */
#define DIT_QUANT_FP8_E4M3 0
#define DIT_QUANT_FP4_E2M1 1        /* FP4, group scales row-major            */
#define DIT_QUANT_FP4_E2M1_128X4 2  /* FP4, group scales in 128x4 tiles       */

/*
 * Token concatenation [a | b] fused with static FP8 or 16-element-group FP4
 * quantisation; the concatenated bf16 row is never written.
 *
 * Defined by: sglang PR 37162 page (the _token_cat_fp8_kernel excerpt under
 * "Key source snippets": a column left of the attention width reads the
 * attention branch, else the MLP branch; values * (1 / scale), clamped to the
 * E4M3 range) and sglang PR 37141 page ("Implementation breakdown" item 1: one
 * 16-element group per GPU thread, packed E2M1 values with one E4M3 scale per
 * group, zero scales for pad rows; the global scale argument is an inverse
 * scale).
 *
 *   kind      DIT_QUANT_FP8_E4M3, DIT_QUANT_FP4_E2M1 (row-major scales) or
 *             DIT_QUANT_FP4_E2M1_128X4 (scales in the 128x4 tile layout, see
 *             DIT_FP4_SCALES_128X4; a_cols + b_cols must be a multiple of 64
 *             and out_scales 16-byte aligned)
 *   out       FP8: [rows, a_cols + b_cols] E4M3 bytes
 *             FP4: [rows, (a_cols + b_cols) / 2] bytes, element 2k in the low
 *             nibble of byte k, element 2k+1 in the high nibble
 *   out_scales  FP4 only (ignored for FP8): [round_up(rows, 128),
 *             (a_cols + b_cols) / 16] E4M3 bytes, row-major; the pad rows
 *             [rows, round_up(rows, 128)) are written as 0x00
 *   a         [rows, a_cols] bf16 (attention branch), in
 *   b         [rows, b_cols] bf16 (MLP branch), in; may be NULL iff b_cols == 0
 *   scale_dev device fp32 scalar. FP8: the static input scale s (codes are
 *             e4m3(clamp(x * (1/s)))). FP4: the global INVERSE scale g; per
 *             group s8 = e4m3(min((amax / 6) * g, 448)), codes
 *             e2m1(x * (g / s8)), all codes 0 when s8 == 0.
 *
 * a_cols and b_cols must be multiples of 16 (a group never straddles the
 * branch boundary) and a_cols >= 16.
 */
int dit_token_cat_quant(int32_t kind, uint8_t* out, uint8_t* out_scales,
                        const void* a, int64_t a_cols, const void* b,
                        int64_t b_cols, int64_t rows, const float* scale_dev,
                        void* stream);

#ifdef __cplusplus
}
#endif
#endif /* DIT_EPILOGUES_H */

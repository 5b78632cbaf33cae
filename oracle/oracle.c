/*
 * oracle.c -- plain, slow, single-threaded CPU oracle for the fused DiT-block
 * epilogues.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark load this library; the GPU library shares
 * nothing with it.
 *
 * Build: gcc -std=c11 -O2 -ffp-contract=off -fno-fast-math -fPIC -shared
 * (x86-64 SSE arithmetic: every float expression below is one IEEE binary32
 * operation, every double expression one IEEE binary64 operation; nothing is
 * contracted into an FMA unless fmaf() is written).
 *
 * Arithmetic model.
 *  1. Where a page prints the operation sequence (the norm/modulate/FP8 loop
 *     of the norm_scale_shift excerpt on the sglang PR 37156 page, the
 *     bias_mul_add excerpt on the sglang PR 37116 page, the token-cat FP8
 *     Triton excerpt on the sglang PR 37162 page), this file performs the same
 *     binary32 steps in the same order. The one fused multiply-add of the
 *     modulation (norm * (1 + scale) + shift, a single fp32 expression that
 *     GPU compilers contract) is written as fmaf().
 *  2. Where no code is printed (LayerNorm and RMSNorm statistics, RoPE, the
 *     gated residual, the FP4 group scale) the value is computed exactly, or in
 *     binary64 to well below binary32 precision, and rounded once at the point
 *     where the split path materialises a tensor.
 *
 * Readings taken where the pages are silent are listed beside each function.
 * Parity unpinned: the FP4 group arithmetic of oracle_token_cat_fp4 against the
 * third-party primitive the sglang PR 37141 page delegates it to (see there).
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ======================================================================== */
/* bfloat16                                                                 */
/* ======================================================================== */

float oracle_f32_from_bf16(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Bit pattern of a value that is already representable in bfloat16 (or is
 * +inf): bfloat16 is the upper half of the binary32 pattern. */
static uint16_t bf16_bits_of_representable(double r) {
    float f = (float)r;
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

/* Distance between adjacent bfloat16 values around m (m >= 0, finite).
 * bfloat16 has 8 significant bits and the binary32 exponent range, so in the
 * binade [2^E, 2^(E+1)) the spacing is 2^(E-7); below 2^-126 (subnormals) it
 * is 2^-133. */
static double bf16_spacing(double m) {
    if (m < 0x1p-126) return 0x1p-133;
    int e;
    (void)frexp(m, &e); /* m = f * 2^e, f in [0.5, 1): binade E = e - 1 */
    return ldexp(1.0, (e - 1) - 7);
}

/* Round the exact real number s + err (|err| <= half an ulp of s, as TwoSum
 * produces) to the nearest bfloat16, ties to even. */
static uint16_t bf16_round(double s, double err) {
    if (isnan(s)) return signbit(s) ? 0xFFC0 : 0x7FC0;
    if (isinf(s)) return signbit(s) ? 0xFF80 : 0x7F80;
    const int neg = signbit(s) ? 1 : 0;
    const double m = fabs(s);          /* magnitude of the binary64 part   */
    const double me = neg ? -err : err; /* exact magnitude is m + me        */
    const double q = bf16_spacing(m);
    const double lo = floor(m / q) * q; /* bf16 value <= m (exact)          */
    const double hi = lo + q;           /* next bf16 value (may be 2^128)   */
    const double mid = lo + 0.5 * q;    /* exactly representable            */
    double r;
    /* m and mid are distinct doubles in one binade, so when m != mid their
     * gap exceeds |me| and m alone decides the side. */
    if (m > mid || (m == mid && me > 0)) {
        r = hi;
    } else if (m < mid || (m == mid && me < 0)) {
        r = lo;
    } else {
        r = (bf16_bits_of_representable(lo) & 1u) ? hi : lo; /* tie: even */
    }
    uint16_t bits = bf16_bits_of_representable(r); /* 2^128 -> +inf */
    return neg ? (uint16_t)(bits | 0x8000u) : bits;
}

uint16_t oracle_bf16_from_f64(double v) { return bf16_round(v, 0.0); }

uint16_t oracle_bf16_from_f32(float v) { return bf16_round((double)v, 0.0); }

uint16_t oracle_bf16_of_exact_sum(double a, double b) {
    /* Knuth's TwoSum: a + b == s + err exactly (no overflow for our data). */
    const double s = a + b;
    const double bv = s - a;
    const double err = (a - (s - bv)) + (b - bv);
    if (s == 0.0) return signbit(s) ? 0x8000 : 0x0000; /* err is 0 here */
    return bf16_round(s, err);
}

/* ======================================================================== */
/* OCP FP8 E4M3FN and E2M1                                                  */
/* ======================================================================== */

/* E4M3FN: sign, 4 exponent bits (bias 7), 3 mantissa bits; no infinities;
 * S.1111.111 is NaN; largest finite magnitude 1.75 * 2^8 = 448 (0x7E). */
double oracle_e4m3_decode(uint8_t code) {
    const int s = code >> 7, e = (code >> 3) & 0xF, m = code & 0x7;
    if (e == 0xF && m == 0x7) return NAN;
    double v = (e == 0) ? ldexp(m / 8.0, -6)          /* subnormal */
                        : ldexp(1.0 + m / 8.0, e - 7); /* normal */
    return s ? -v : v;
}

uint8_t oracle_e4m3_encode(float v) {
    if (isnan(v)) return 0x7F;
    const uint8_t sign = signbit(v) ? 0x80 : 0x00;
    const double m = fabs((double)v);
    if (m >= 448.0) return (uint8_t)(sign | 0x7E); /* saturate */
    /* Non-negative codes 0x00..0x7E have strictly increasing values. Find the
     * largest code whose value is <= m, keeping value(lo) <= m < value(hi). */
    int lo = 0, hi = 0x7E;
    while (hi - lo > 1) {
        const int mid = (lo + hi) / 2;
        if (oracle_e4m3_decode((uint8_t)mid) <= m) lo = mid; else hi = mid;
    }
    const double midpoint =
        0.5 * (oracle_e4m3_decode((uint8_t)lo) + oracle_e4m3_decode((uint8_t)hi));
    int c;
    if (m < midpoint) c = lo;
    else if (m > midpoint) c = hi;
    else c = (lo & 1) ? hi : lo; /* tie: even code (even mantissa) */
    return (uint8_t)(sign | c);
}

/* E2M1: sign, 2 exponent bits, 1 mantissa bit. Codes 0..7 hold the
 * magnitudes below; 8..15 are the negatives. */
static const double kE2M1Magnitude[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double oracle_e2m1_decode(uint8_t code) {
    const double v = kE2M1Magnitude[code & 7];
    return (code & 8) ? -v : v;
}

uint8_t oracle_e2m1_encode(float v) {
    const uint8_t sign = signbit(v) ? 0x8 : 0x0;
    const double m = fabs((double)v);
    if (m >= 6.0) return (uint8_t)(sign | 7); /* saturate */
    int lo = 0; /* largest code with magnitude <= m */
    while (lo < 7 && kE2M1Magnitude[lo + 1] <= m) ++lo;
    const int hi = lo + 1;
    const double midpoint = 0.5 * (kE2M1Magnitude[lo] + kE2M1Magnitude[hi]);
    int c;
    if (m < midpoint) c = lo;
    else if (m > midpoint) c = hi;
    else c = (lo & 1) ? hi : lo; /* tie: even code */
    return (uint8_t)(sign | c);
}

void oracle_bf16_from_f32_n(const float* in, uint16_t* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_bf16_from_f32(in[i]);
}
void oracle_bf16_from_f64_n(const double* in, uint16_t* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_bf16_from_f64(in[i]);
}
void oracle_bf16_of_exact_sum_n(const double* a, const double* b, uint16_t* out,
                                int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_bf16_of_exact_sum(a[i], b[i]);
}
void oracle_e4m3_encode_n(const float* in, uint8_t* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_encode(in[i]);
}
void oracle_e2m1_encode_n(const float* in, uint8_t* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_e2m1_encode(in[i]);
}

/* ======================================================================== */
/* Row statistics                                                           */
/* ======================================================================== */

static float bf(uint16_t h) { return oracle_f32_from_bf16(h); }

/* LayerNorm without affine, statistics in fp32 (sglang PR 37156 page,
 * "Implementation breakdown" item 1 and the norm_scale_shift excerpt, which
 * uses a per-row mean and a per-row factor 1/sqrt(var + eps) in fp32; the
 * formula for them is not printed). Reading: two-pass mean and biased
 * variance in binary64 over the exact bf16 inputs, each rounded once to
 * binary32. */
void oracle_layernorm_stats(const uint16_t* v, int64_t n, float eps,
                            float* mean32, float* factor32) {
    double sum = 0.0;
    for (int64_t i = 0; i < n; ++i) sum += (double)bf(v[i]);
    const double mean = sum / (double)n;
    double ss = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        const double d = (double)bf(v[i]) - mean;
        ss += d * d;
    }
    const double var = ss / (double)n;
    *mean32 = (float)mean;
    *factor32 = (float)(1.0 / sqrt(var + (double)eps));
}

/* Per-head RMSNorm inverse (sglang PR 37123 page, "Implementation breakdown"
 * item 3: warp-reduced RMS per head). Reading: mean of squares in binary64,
 * 1/sqrt(ms + eps) rounded once to binary32. */
float oracle_rms_inverse(const uint16_t* v, int64_t n, float eps) {
    double ss = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        const double x = (double)bf(v[i]);
        ss += x * x;
    }
    const double ms = ss / (double)n;
    return (float)(1.0 / sqrt(ms + (double)eps));
}

/* ======================================================================== */
/* LayerNorm + AdaLN modulation + static FP8 (sglang PR 37156 page)         */
/* ======================================================================== */

/* One row, following the kQuantizeFp8 loop of the norm_scale_shift excerpt
 * ("Key source snippets"): norm = bf16((v - mean) * factor); y = bf16(norm *
 * (1 + scale) + shift). */
static void norm_modulate_row(uint16_t* y, const uint16_t* v, const uint16_t* scale,
                              const uint16_t* shift, int64_t hidden, float eps) {
    float mean, factor;
    oracle_layernorm_stats(v, hidden, eps, &mean, &factor);
    for (int64_t j = 0; j < hidden; ++j) {
        const float d = bf(v[j]) - mean;
        const float t = d * factor;
        const float norm = bf(oracle_bf16_from_f32(t));
        const float one_plus_scale = 1.0f + bf(scale[j]);
        const float modulated = fmaf(norm, one_plus_scale, bf(shift[j]));
        y[j] = oracle_bf16_from_f32(modulated);
    }
}

/* The same excerpt's FP8 step on one row of y: q = e4m3(clamp(y * (1 /
 * input_scale), +-448)). The reciprocal is IEEE binary32 division (the page's
 * NVIDIA-specific reciprocal instruction is not reproduced). */
static void fp8_quantize_row(uint8_t* q, float* q_pre, const uint16_t* y, float inv,
                             int64_t hidden) {
    for (int64_t j = 0; j < hidden; ++j) {
        const float scaled = bf(y[j]) * inv;
        const float clamped = fminf(fmaxf(scaled, -448.0f), 448.0f);
        q[j] = oracle_e4m3_encode(clamped);
        if (q_pre) q_pre[j] = clamped;
    }
}

static void norm_modulate_fp8_row(uint16_t* y, uint8_t* q, float* q_pre,
                                  const uint16_t* v, const uint16_t* scale,
                                  const uint16_t* shift, float inv,
                                  int64_t hidden, float eps) {
    norm_modulate_row(y, v, scale, shift, hidden, eps);
    fp8_quantize_row(q, q_pre, y, inv, hidden);
}

void oracle_norm_modulate_fp8(uint16_t* y, uint8_t* q, float* q_pre,
                              const uint16_t* x, const uint16_t* scale,
                              const uint16_t* shift, float input_scale,
                              int64_t rows, int64_t hidden, float eps) {
    const float inv = 1.0f / input_scale;
    for (int64_t r = 0; r < rows; ++r) {
        norm_modulate_fp8_row(y + r * hidden, q + r * hidden,
                              q_pre ? q_pre + r * hidden : NULL, x + r * hidden,
                              scale, shift, inv, hidden, eps);
    }
}

/* Optional input bias and gated residual before the same norm (sglang PR 37156
 * page: the residual variant also returns residual_out; sglang PR 37116 page,
 * "Implementation breakdown" item 3: x + bias is folded into the same kernel,
 * and the fallback first forms a BF16 x + bias). Readings: the bias add is
 * rounded to bf16 (as the fallback materialises it); residual + gate * xb is
 * rounded ONCE to bf16, the same single-rounding rule the bias_mul_add
 * excerpt states for its gated multiply-add. gate * xb is exact in binary64
 * (8 x 8 significant bits). */
static void gated_residual_row(uint16_t* rr, const uint16_t* xr, const uint16_t* bias,
                               const uint16_t* gate, const uint16_t* resr, int64_t hidden) {
    for (int64_t j = 0; j < hidden; ++j) {
        float xb = bf(xr[j]);
        if (bias) xb = bf(oracle_bf16_from_f32(xb + bf(bias[j])));
        const double product = (double)bf(gate[j]) * (double)xb;
        rr[j] = oracle_bf16_of_exact_sum(product, (double)bf(resr[j]));
    }
}

void oracle_scale_residual_norm_modulate_fp8(
    uint16_t* r_out, uint16_t* y, uint8_t* q, float* q_pre,
    const uint16_t* x, const uint16_t* bias, const uint16_t* gate,
    const uint16_t* residual, const uint16_t* scale, const uint16_t* shift,
    float input_scale, int64_t rows, int64_t hidden, float eps) {
    const float inv = 1.0f / input_scale;
    for (int64_t r = 0; r < rows; ++r) {
        uint16_t* rr = r_out + r * hidden;
        gated_residual_row(rr, x + r * hidden, bias, gate, residual + r * hidden, hidden);
        norm_modulate_fp8_row(y + r * hidden, q + r * hidden,
                              q_pre ? q_pre + r * hidden : NULL, rr, scale,
                              shift, inv, hidden, eps);
    }
}

/* ======================================================================== */
/* QKV epilogue (sglang PR 37123 page)                                      */
/* ======================================================================== */

/* One head of Q or K: RMSNorm with weight, then interleaved RoPE.
 * Readings: the normalised head is rounded to bf16 before RoPE (the split
 * path materialises it, and the fused kernel is stated to be bit-exact to
 * that path: "Implementation breakdown" items 3 and 5); RoPE is interleaved
 * (is_neox=False in the fallback excerpt), pair (2i, 2i+1) rotated by +angle:
 * (n0*c - n1*s, n1*c + n0*s), each output one exact rounding to bf16 (the
 * products bf16 x fp32 are exact in binary64). */
static void qk_norm_rope_head(uint16_t* out, const uint16_t* x,
                              const uint16_t* w, const float* cos_row,
                              const float* sin_row, int32_t head_dim,
                              float eps, uint16_t* scratch) {
    const float inv = oracle_rms_inverse(x, head_dim, eps);
    for (int32_t i = 0; i < head_dim; ++i) {
        const float t = bf(x[i]) * inv;
        scratch[i] = oracle_bf16_from_f32(t * bf(w[i]));
    }
    for (int32_t p = 0; p < head_dim / 2; ++p) {
        const double n0 = (double)bf(scratch[2 * p]);
        const double n1 = (double)bf(scratch[2 * p + 1]);
        const double c = (double)cos_row[p];
        const double s = (double)sin_row[p];
        out[2 * p] = oracle_bf16_of_exact_sum(n0 * c, -(n1 * s));
        out[2 * p + 1] = oracle_bf16_of_exact_sum(n1 * c, n0 * s);
    }
}

/* Joint order is [text, image] (join_seqs(txt, img) in the fallback excerpt):
 * joint row j < txt_rows comes from text row j, the rest from image row
 * j - txt_rows. V is copied unchanged. */
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
    int32_t heads, int32_t head_dim, float img_eps, float txt_eps) {
    uint16_t* scratch = (uint16_t*)malloc((size_t)head_dim * sizeof(uint16_t));
    const int64_t half = head_dim / 2;
    for (int64_t j = 0; j < txt_rows + img_rows; ++j) {
        const int is_txt = j < txt_rows;
        const int64_t i = is_txt ? j : j - txt_rows;
        const int64_t stride = is_txt ? txt_row_stride : img_row_stride;
        const uint16_t* qs = (is_txt ? txt_q : img_q) + i * stride;
        const uint16_t* ks = (is_txt ? txt_k : img_k) + i * stride;
        const uint16_t* vs = (is_txt ? txt_v : img_v) + i * stride;
        const uint16_t* qw = is_txt ? txt_q_w : img_q_w;
        const uint16_t* kw = is_txt ? txt_k_w : img_k_w;
        const float* cr = (is_txt ? txt_cos : img_cos) + i * half;
        const float* sr = (is_txt ? txt_sin : img_sin) + i * half;
        const float eps = is_txt ? txt_eps : img_eps;
        for (int32_t h = 0; h < heads; ++h) {
            const int64_t out_off = (j * heads + h) * head_dim;
            qk_norm_rope_head(joint_q + out_off, qs + (int64_t)h * head_dim, qw,
                              cr, sr, head_dim, eps, scratch);
            qk_norm_rope_head(joint_k + out_off, ks + (int64_t)h * head_dim, kw,
                              cr, sr, head_dim, eps, scratch);
            memcpy(joint_v + out_off, vs + (int64_t)h * head_dim,
                   (size_t)head_dim * sizeof(uint16_t));
        }
    }
    free(scratch);
}

/* ======================================================================== */
/* bias_mul_add (sglang PR 37116 page)                                      */
/* ======================================================================== */

/* bias_mul_add excerpt ("Key source snippets"): the bias add is rounded to
 * bf16, then a native bf16 fused multiply-add forms biased * gate + residual
 * with a single rounding. The product of two bf16 values is exact in
 * binary64, so the single rounding is bf16 of an exact two-term sum. */
void oracle_bias_mul_add(uint16_t* y, const uint16_t* x, const uint16_t* bias,
                         const uint16_t* gate, const uint16_t* residual,
                         int64_t rows, int64_t hidden) {
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t j = 0; j < hidden; ++j) {
            const int64_t o = r * hidden + j;
            const float b = bias ? bf(oracle_bf16_from_f32(bf(x[o]) + bf(bias[j])))
                                 : bf(x[o]);
            const double product = (double)b * (double)bf(gate[j]);
            y[o] = oracle_bf16_of_exact_sum(product, (double)bf(residual[o]));
        }
    }
}

/* ======================================================================== */
/* Token concatenation + quantisation (sglang PR 37162 and PR 37141 pages)  */
/* ======================================================================== */

/* The concatenated row [a | b], built explicitly. */
static void cat_row(uint16_t* dst, const uint16_t* a, int64_t a_cols,
                    const uint16_t* b, int64_t b_cols, int64_t r) {
    memcpy(dst, a + r * a_cols, (size_t)a_cols * sizeof(uint16_t));
    if (b_cols) memcpy(dst + a_cols, b + r * b_cols, (size_t)b_cols * sizeof(uint16_t));
}

/* Token-cat FP8 Triton excerpt (sglang PR 37162 page): each output column
 * takes the attention value if it is left of the attention width, else the
 * MLP value; then clamp(value * (1.0 / scale), FP8_MIN, FP8_MAX) -> E4M3. */
void oracle_token_cat_fp8(uint8_t* out, float* pre, const uint16_t* a,
                          int64_t a_cols, const uint16_t* b, int64_t b_cols,
                          int64_t rows, float input_scale) {
    const int64_t cols = a_cols + b_cols;
    const float inv = 1.0f / input_scale;
    uint16_t* row = (uint16_t*)malloc((size_t)(cols ? cols : 1) * sizeof(uint16_t));
    for (int64_t r = 0; r < rows; ++r) {
        cat_row(row, a, a_cols, b, b_cols, r);
        for (int64_t c = 0; c < cols; ++c) {
            const float scaled = bf(row[c]) * inv;
            const float clamped = fminf(fmaxf(scaled, -448.0f), 448.0f);
            out[r * cols + c] = oracle_e4m3_encode(clamped);
            if (pre) pre[r * cols + c] = clamped;
        }
    }
    free(row);
}

/* 16-element-group FP4 (sglang PR 37141 page, "Implementation breakdown"
 * item 1: one group of 16 elements per GPU thread, packed E2M1 values plus one
 * E4M3 scale per group, pad rows get a zero scale; the global scale argument
 * is an inverse scale, input_scale_inv). The page delegates the per-group
 * arithmetic to a third-party primitive; readings:
 *   s_pre = RN32(RN32(amax / 6) * g); s8 = e4m3(min(s_pre, 448));
 *   k = RN32(g / dec(s8)) (zero scale -> every code +0);
 *   code = e2m1(RN32(x * k)); byte j = code(2j) | code(2j+1) << 4.
 * Scales are row-major [round_up(rows, 128), cols / 16].
 * Pinned by closed forms (exactly representable groups, zero and saturating
 * groups, the dequantisation error bound); parity with the page's third-party
 * primitive itself is unpinned, since the page shows none of its outputs. */
static void fp4_quantize_row(uint8_t* packed, uint8_t* scales, float* s_pre, float* pre,
                             const uint16_t* row, int64_t cols, float g) {
    for (int64_t gi = 0; gi < cols / 16; ++gi) {
        const uint16_t* grp = row + gi * 16;
        float amax = 0.0f;
        for (int k = 0; k < 16; ++k) amax = fmaxf(amax, fabsf(bf(grp[k])));
        const float sp = (amax / 6.0f) * g;
        const uint8_t s8 = oracle_e4m3_encode(fminf(sp, 448.0f));
        const float kscale = (s8 == 0) ? 0.0f : g / (float)oracle_e4m3_decode(s8);
        uint8_t codes[16];
        for (int k = 0; k < 16; ++k) {
            const float t = bf(grp[k]) * kscale;
            codes[k] = (s8 == 0) ? 0 : oracle_e2m1_encode(t);
            if (pre) pre[gi * 16 + k] = t;
        }
        for (int k = 0; k < 8; ++k)
            packed[gi * 8 + k] = (uint8_t)(codes[2 * k] | (codes[2 * k + 1] << 4));
        scales[gi] = s8;
        if (s_pre) s_pre[gi] = sp;
    }
}

void oracle_token_cat_fp4(uint8_t* packed, uint8_t* scales, float* s_pre,
                          float* pre, const uint16_t* a, int64_t a_cols,
                          const uint16_t* b, int64_t b_cols, int64_t rows,
                          float g) {
    const int64_t cols = a_cols + b_cols;
    const int64_t groups = cols / 16;
    const int64_t rows_padded = ((rows + 127) / 128) * 128;
    memset(scales, 0, (size_t)(rows_padded * groups));
    uint16_t* row = (uint16_t*)malloc((size_t)(cols ? cols : 1) * sizeof(uint16_t));
    for (int64_t r = 0; r < rows; ++r) {
        cat_row(row, a, a_cols, b, b_cols, r);
        fp4_quantize_row(packed + r * (cols / 2), scales + r * groups,
                         s_pre ? s_pre + r * groups : NULL, pre ? pre + r * cols : NULL,
                         row, cols, g);
    }
    free(row);
}

/* ======================================================================== */
/* NVFP4 output on the LayerNorm path                                       */
/* ======================================================================== */

/* The (residual-)norm variants with NVFP4 instead of FP8 output. The pages
 * only name this fusion (the Qwen-Image residual norm + NVFP4 PR, listed
 * among the related PRs of the sglang PR 37123 and PR 37162 pages). Reading:
 * the bf16 y of the FP8 variants, quantised exactly as the token-cat FP4
 * output of the sglang PR 37141 page (16-element groups, E4M3 scale from the
 * global inverse scale g, row-major scales, pad rows to a multiple of 128
 * with zero scales). */
void oracle_norm_modulate_fp4(uint16_t* y, uint8_t* packed, uint8_t* scales,
                              float* s_pre, float* pre, const uint16_t* x,
                              const uint16_t* scale, const uint16_t* shift,
                              float g, int64_t rows, int64_t hidden, float eps) {
    const int64_t groups = hidden / 16;
    const int64_t rows_padded = ((rows + 127) / 128) * 128;
    memset(scales, 0, (size_t)(rows_padded * groups));
    for (int64_t r = 0; r < rows; ++r) {
        norm_modulate_row(y + r * hidden, x + r * hidden, scale, shift, hidden, eps);
        fp4_quantize_row(packed + r * (hidden / 2), scales + r * groups,
                         s_pre ? s_pre + r * groups : NULL, pre ? pre + r * hidden : NULL,
                         y + r * hidden, hidden, g);
    }
}

void oracle_scale_residual_norm_modulate_fp4(
    uint16_t* r_out, uint16_t* y, uint8_t* packed, uint8_t* scales, float* s_pre,
    float* pre, const uint16_t* x, const uint16_t* bias, const uint16_t* gate,
    const uint16_t* residual, const uint16_t* scale, const uint16_t* shift,
    float g, int64_t rows, int64_t hidden, float eps) {
    for (int64_t r = 0; r < rows; ++r)
        gated_residual_row(r_out + r * hidden, x + r * hidden, bias, gate,
                           residual + r * hidden, hidden);
    oracle_norm_modulate_fp4(y, packed, scales, s_pre, pre, r_out, scale, shift, g, rows,
                             hidden, eps);
}

/* ======================================================================== */
/* FP4 scale layout for FP4 GEMMs                                           */
/* ======================================================================== */

/* The 128x4 interleaved ("swizzled") scale layout the sglang PR 37141 page
 * names for its NVFP4 output (get_sf_out_offset_128x4, matching FlashInfer)
 * without spelling it out. Reading, from the public description of this
 * block-scale layout for FP4 GEMMs: the [rows_padded, groups] scale matrix
 * (rows_padded a multiple of 128, groups a multiple of 4) is cut into tiles
 * of 128 rows x 4 columns, stored one after another, the tile column index
 * fastest; inside a tile, row m and column k go to byte
 * (m % 32) * 16 + (m / 32) * 4 + k, i.e. the tile is [32][4][4] over
 * (m % 32, m / 32, k). Parity unpinned against the third-party layout itself:
 * the pages print none of its bytes. */
void oracle_fp4_scales_to_128x4(uint8_t* out, const uint8_t* row_major,
                                int64_t rows_padded, int64_t groups) {
    const int64_t tiles_per_row = groups / 4;
    for (int64_t m = 0; m < rows_padded; ++m) {
        for (int64_t k = 0; k < groups; ++k) {
            const int64_t tile = (m / 128) * tiles_per_row + k / 4;
            const int64_t r = m % 128;
            const int64_t inner = (r % 32) * 16 + (r / 32) * 4 + k % 4;
            out[tile * 512 + inner] = row_major[m * groups + k];
        }
    }
}

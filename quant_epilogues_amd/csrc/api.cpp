// api.cpp -- the C ABI of libdit_epilogues (declared in include/dit_epilogues.h).
//
// Each entry point validates its arguments on the host (pointers, sizes,
// alignment, supported shapes) before touching HIP, so a refusal enqueues
// nothing and leaves outputs untouched; it then fills the kernel argument
// block and enqueues one kernel on the caller's stream. Nothing here
// allocates, frees, copies or synchronises.
#include "dit_epilogues.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "kernels.h"

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return status;
}

int ok() {
    g_last_error[0] = '\0';
    return DIT_OK;
}

bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

// Discard an error left by an earlier, unrelated HIP call on this thread so
// that the status read after our launch is our own.
void clear_stale_hip_error() { (void)hipGetLastError(); }

int launched(hipError_t e, const char* what) {
    if (e == dit::kGridTooLarge)
        return fail(DIT_ERR_UNSUPPORTED, "%s: too large for one launch (grid limit of 2^32 lanes)", what);
    if (e != hipSuccess) return fail(DIT_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
    return ok();
}

// Coarse bound that keeps row arithmetic (padding to 128 rows, products with
// row widths) far from overflow; the launchers check the exact grid limit.
constexpr int64_t kMaxRows = (int64_t(1) << 31) - 128;

}  // namespace

extern "C" {

int dit_abi_version(void) { return DIT_ABI_VERSION; }

const char* dit_status_string(int status) {
    switch (status) {
        case DIT_OK: return "DIT_OK";
        case DIT_ERR_NULL: return "DIT_ERR_NULL";
        case DIT_ERR_SHAPE: return "DIT_ERR_SHAPE";
        case DIT_ERR_ALIGN: return "DIT_ERR_ALIGN";
        case DIT_ERR_UNSUPPORTED: return "DIT_ERR_UNSUPPORTED";
        case DIT_ERR_HIP: return "DIT_ERR_HIP";
        default: return "DIT_ERR_UNKNOWN";
    }
}

const char* dit_last_error(void) { return g_last_error; }

static int check_norm_shape(const char* fn, int64_t rows, int64_t hidden) {
    if (rows < 0 || hidden <= 0)
        return fail(DIT_ERR_SHAPE, "%s: rows (%lld) must be >= 0 and hidden (%lld) > 0", fn,
                    (long long)rows, (long long)hidden);
    if (hidden % 8 != 0 || hidden > dit::kMaxHidden)
        return fail(DIT_ERR_UNSUPPORTED, "%s: hidden (%lld) must be a multiple of 8 and <= %d", fn,
                    (long long)hidden, dit::kMaxHidden);
    if (rows > kMaxRows) return fail(DIT_ERR_UNSUPPORTED, "%s: rows (%lld) too large", fn, (long long)rows);
    return DIT_OK;
}

int dit_norm_modulate_fp8(void* y, uint8_t* q, const void* x, const void* scale,
                          const void* shift, const float* input_scale_dev, int64_t rows,
                          int64_t hidden, float eps, void* stream) {
    const char* fn = "dit_norm_modulate_fp8";
    if (!x || !scale || !shift || (!y && !q) || (q && !input_scale_dev))
        return fail(DIT_ERR_NULL, "%s: a required pointer is NULL (y and q may not both be NULL; "
                    "q needs input_scale)", fn);
    if (int st = check_norm_shape(fn, rows, hidden)) return st;
    if (!aligned(y, 16) || !aligned(q, 16) || !aligned(x, 16) || !aligned(scale, 16) ||
        !aligned(shift, 16) || !aligned(input_scale_dev, 4))
        return fail(DIT_ERR_ALIGN, "%s: tensors must be 16-byte aligned (input_scale 4-byte)", fn);
    if (rows == 0) return ok();
    dit::NormModulateArgs a{};
    a.y = static_cast<uint16_t*>(y);
    a.q = q;
    a.x = static_cast<const uint16_t*>(x);
    a.scale = static_cast<const uint16_t*>(scale);
    a.shift = static_cast<const uint16_t*>(shift);
    a.input_scale = input_scale_dev;
    a.rows = rows;
    a.hidden = (int32_t)hidden;
    a.eps = eps;
    clear_stale_hip_error();
    return launched(dit::launch_norm_modulate_fp8(a, static_cast<hipStream_t>(stream)), fn);
}

// Host checks of one stream of dit_norm_modulate_fp8_dual; fills `a`.
static int dual_stream(const char* fn, const char* which, dit::NormModulateArgs& a, void* y,
                       uint8_t* q, const void* x, const void* scale, const void* shift,
                       const float* input_scale_dev, int64_t rows, int64_t hidden, float eps) {
    if (rows < 0) return fail(DIT_ERR_SHAPE, "%s: %s_rows (%lld) must be >= 0", fn, which, (long long)rows);
    if (rows > 0 && (!x || !scale || !shift || (!y && !q) || (q && !input_scale_dev)))
        return fail(DIT_ERR_NULL, "%s: a required %s pointer is NULL (y and q may not both be NULL; "
                    "q needs input_scale)", fn, which);
    if (rows > 0 && (!aligned(y, 16) || !aligned(q, 16) || !aligned(x, 16) || !aligned(scale, 16) ||
                     !aligned(shift, 16) || !aligned(input_scale_dev, 4)))
        return fail(DIT_ERR_ALIGN, "%s: %s tensors must be 16-byte aligned (input_scale 4-byte)", fn,
                    which);
    a = dit::NormModulateArgs{};
    a.y = static_cast<uint16_t*>(y);
    a.q = q;
    a.x = static_cast<const uint16_t*>(x);
    a.scale = static_cast<const uint16_t*>(scale);
    a.shift = static_cast<const uint16_t*>(shift);
    a.input_scale = input_scale_dev;
    a.rows = rows;
    a.hidden = (int32_t)hidden;
    a.eps = eps;
    return DIT_OK;
}

int dit_norm_modulate_fp8_dual(void* img_y, uint8_t* img_q, const void* img_x,
                               const void* img_scale, const void* img_shift,
                               const float* img_input_scale_dev, int64_t img_rows, float img_eps,
                               void* txt_y, uint8_t* txt_q, const void* txt_x,
                               const void* txt_scale, const void* txt_shift,
                               const float* txt_input_scale_dev, int64_t txt_rows, float txt_eps,
                               int64_t hidden, void* stream) {
    const char* fn = "dit_norm_modulate_fp8_dual";
    if (img_rows < 0 || txt_rows < 0)
        return fail(DIT_ERR_SHAPE, "%s: row counts must be >= 0", fn);
    if (img_rows > kMaxRows || txt_rows > kMaxRows)  // keeps the sum below from overflowing
        return fail(DIT_ERR_UNSUPPORTED, "%s: row counts too large", fn);
    if (int st = check_norm_shape(fn, img_rows + txt_rows, hidden)) return st;
    dit::NormModulateArgs img, txt;
    if (int st = dual_stream(fn, "img", img, img_y, img_q, img_x, img_scale, img_shift,
                             img_input_scale_dev, img_rows, hidden, img_eps))
        return st;
    if (int st = dual_stream(fn, "txt", txt, txt_y, txt_q, txt_x, txt_scale, txt_shift,
                             txt_input_scale_dev, txt_rows, hidden, txt_eps))
        return st;
    if (img_rows + txt_rows == 0) return ok();
    clear_stale_hip_error();
    // Text rows first, then image rows (the joint order of the QKV epilogue).
    return launched(dit::launch_norm_modulate_fp8_dual(txt, img, static_cast<hipStream_t>(stream)), fn);
}

int dit_scale_residual_norm_modulate_fp8(void* residual_out, void* y, uint8_t* q, const void* x,
                                         const void* bias, const void* gate,
                                         const void* residual, const void* scale,
                                         const void* shift, const float* input_scale_dev,
                                         int64_t rows, int64_t hidden, float eps, void* stream) {
    const char* fn = "dit_scale_residual_norm_modulate_fp8";
    if (!residual_out || !x || !gate || !residual || !scale || !shift || (!y && !q) ||
        (q && !input_scale_dev))
        return fail(DIT_ERR_NULL, "%s: a required pointer is NULL (y and q may not both be NULL; "
                    "q needs input_scale)", fn);
    if (int st = check_norm_shape(fn, rows, hidden)) return st;
    if (!aligned(residual_out, 16) || !aligned(y, 16) || !aligned(q, 16) || !aligned(x, 16) ||
        (bias && !aligned(bias, 16)) || !aligned(gate, 16) || !aligned(residual, 16) ||
        !aligned(scale, 16) || !aligned(shift, 16) || !aligned(input_scale_dev, 4))
        return fail(DIT_ERR_ALIGN, "%s: tensors must be 16-byte aligned (input_scale 4-byte)", fn);
    if (rows == 0) return ok();
    dit::NormModulateArgs a{};
    a.y = static_cast<uint16_t*>(y);
    a.q = q;
    a.r_out = static_cast<uint16_t*>(residual_out);
    a.x = static_cast<const uint16_t*>(x);
    a.residual = static_cast<const uint16_t*>(residual);
    a.bias = static_cast<const uint16_t*>(bias);
    a.gate = static_cast<const uint16_t*>(gate);
    a.scale = static_cast<const uint16_t*>(scale);
    a.shift = static_cast<const uint16_t*>(shift);
    a.input_scale = input_scale_dev;
    a.rows = rows;
    a.hidden = (int32_t)hidden;
    a.eps = eps;
    clear_stale_hip_error();
    return launched(dit::launch_norm_modulate_fp8(a, static_cast<hipStream_t>(stream)), fn);
}

static int launch_norm_fp4(const char* fn, void* residual_out, void* y, uint8_t* packed,
                           uint8_t* scales, int32_t scale_layout, const void* x,
                           const void* bias, const void* gate,
                           const void* residual, const void* scale, const void* shift,
                           const float* g_dev, int64_t rows, int64_t hidden, float eps,
                           void* stream) {
    if (int st = check_norm_shape(fn, rows, hidden)) return st;
    if (hidden % 16 != 0)
        return fail(DIT_ERR_UNSUPPORTED, "%s: hidden (%lld) must be a multiple of 16 (FP4 groups)",
                    fn, (long long)hidden);
    if (scale_layout != DIT_FP4_SCALES_ROW_MAJOR && scale_layout != DIT_FP4_SCALES_128X4)
        return fail(DIT_ERR_UNSUPPORTED, "%s: unknown scale layout %d", fn, scale_layout);
    if (scale_layout == DIT_FP4_SCALES_128X4 && hidden % 64 != 0)
        return fail(DIT_ERR_UNSUPPORTED, "%s: the 128x4 scale layout needs hidden %% 64 == 0", fn);
    if (!aligned(y, 16) || !aligned(packed, 16) || !aligned(x, 16) || (bias && !aligned(bias, 16)) ||
        !aligned(gate, 16) || !aligned(residual, 16) || !aligned(residual_out, 16) ||
        !aligned(scale, 16) || !aligned(shift, 16) || !aligned(g_dev, 4))
        return fail(DIT_ERR_ALIGN, "%s: tensors must be 16-byte aligned (scales: any; g 4-byte)", fn);
    if (rows == 0) return ok();
    dit::NormModulateArgs a{};
    a.y = static_cast<uint16_t*>(y);
    a.q = nullptr;
    a.r_out = static_cast<uint16_t*>(residual_out);
    a.x = static_cast<const uint16_t*>(x);
    a.residual = static_cast<const uint16_t*>(residual);
    a.bias = static_cast<const uint16_t*>(bias);
    a.gate = static_cast<const uint16_t*>(gate);
    a.scale = static_cast<const uint16_t*>(scale);
    a.shift = static_cast<const uint16_t*>(shift);
    a.input_scale = g_dev;
    a.fp4 = packed;
    a.fp4_scales = scales;
    a.fp4_rows_padded = (rows + 127) / 128 * 128;
    a.fp4_tiled = scale_layout == DIT_FP4_SCALES_128X4;
    a.rows = rows;
    a.hidden = (int32_t)hidden;
    a.eps = eps;
    clear_stale_hip_error();
    return launched(dit::launch_norm_modulate_fp8(a, static_cast<hipStream_t>(stream)), fn);
}

int dit_norm_modulate_fp4(void* y, uint8_t* packed, uint8_t* scales, int32_t scale_layout,
                          const void* x, const void* scale, const void* shift,
                          const float* global_scale_dev, int64_t rows, int64_t hidden,
                          float eps, void* stream) {
    const char* fn = "dit_norm_modulate_fp4";
    if (!packed || !scales || !x || !scale || !shift || !global_scale_dev)
        return fail(DIT_ERR_NULL, "%s: a required pointer is NULL", fn);
    return launch_norm_fp4(fn, nullptr, y, packed, scales, scale_layout, x, nullptr, nullptr,
                           nullptr, scale, shift, global_scale_dev, rows, hidden, eps, stream);
}

int dit_scale_residual_norm_modulate_fp4(void* residual_out, void* y, uint8_t* packed,
                                         uint8_t* scales, int32_t scale_layout,
                                         const void* x, const void* bias,
                                         const void* gate, const void* residual,
                                         const void* scale, const void* shift,
                                         const float* global_scale_dev, int64_t rows,
                                         int64_t hidden, float eps, void* stream) {
    const char* fn = "dit_scale_residual_norm_modulate_fp4";
    if (!residual_out || !packed || !scales || !x || !gate || !residual || !scale || !shift ||
        !global_scale_dev)
        return fail(DIT_ERR_NULL, "%s: a required pointer is NULL", fn);
    return launch_norm_fp4(fn, residual_out, y, packed, scales, scale_layout, x, bias, gate,
                           residual, scale, shift, global_scale_dev, rows, hidden, eps, stream);
}

int dit_qkv_epilogue(void* joint_q, void* joint_k, void* joint_v, const void* img_q,
                     const void* img_k, const void* img_v, int64_t img_rows,
                     int64_t img_row_stride, const void* txt_q, const void* txt_k,
                     const void* txt_v, int64_t txt_rows, int64_t txt_row_stride,
                     const void* img_q_w, const void* img_k_w, const void* txt_q_w,
                     const void* txt_k_w, const float* img_cos, const float* img_sin,
                     const float* txt_cos, const float* txt_sin, int64_t rope_row_stride,
                     int32_t heads, int32_t head_dim, float img_eps, float txt_eps,
                     void* stream) {
    const char* fn = "dit_qkv_epilogue";
    if (img_rows < 0 || txt_rows < 0)
        return fail(DIT_ERR_SHAPE, "%s: row counts must be >= 0", fn);
    if (!joint_q || !joint_k || !joint_v)
        return fail(DIT_ERR_NULL, "%s: a joint output pointer is NULL", fn);
    if (img_rows > 0 && (!img_q || !img_k || !img_v || !img_q_w || !img_k_w || !img_cos || !img_sin))
        return fail(DIT_ERR_NULL, "%s: an image-stream pointer is NULL", fn);
    if (txt_rows > 0 && (!txt_q || !txt_k || !txt_v || !txt_q_w || !txt_k_w || !txt_cos || !txt_sin))
        return fail(DIT_ERR_NULL, "%s: a text-stream pointer is NULL", fn);
    if (head_dim != dit::kHeadDim)
        return fail(DIT_ERR_UNSUPPORTED, "%s: head_dim %d is not supported (only %d)", fn, head_dim,
                    dit::kHeadDim);
    if (heads < 1 || heads > dit::kMaxHeads)
        return fail(DIT_ERR_UNSUPPORTED, "%s: heads %d outside [1, %d]", fn, heads, dit::kMaxHeads);
    const int64_t width = (int64_t)heads * head_dim;
    if ((img_rows > 0 && (img_row_stride < width || img_row_stride % 8 != 0)) ||
        (txt_rows > 0 && (txt_row_stride < width || txt_row_stride % 8 != 0)))
        return fail(DIT_ERR_SHAPE, "%s: row strides must be >= heads*head_dim (%lld) and a multiple of 8",
                    fn, (long long)width);
    if (rope_row_stride < head_dim / 2 || rope_row_stride % 4 != 0)
        return fail(DIT_ERR_SHAPE, "%s: rope_row_stride (%lld) must be >= head_dim/2 and a multiple of 4",
                    fn, (long long)rope_row_stride);
    const int64_t hblocks = (heads + dit::kQkvHeadsPerWave - 1) / dit::kQkvHeadsPerWave;
    if (img_rows > kMaxRows || txt_rows > kMaxRows || (img_rows + txt_rows) * hblocks >= (int64_t(1) << 32) - 4)
        return fail(DIT_ERR_UNSUPPORTED, "%s: too many tokens", fn);
    const void* ptrs16[] = {joint_q, joint_k, joint_v};
    for (const void* p : ptrs16)
        if (!aligned(p, 16)) return fail(DIT_ERR_ALIGN, "%s: outputs must be 16-byte aligned", fn);
    if (img_rows > 0) {
        const void* ps[] = {img_q, img_k, img_v, img_q_w, img_k_w, img_cos, img_sin};
        for (const void* p : ps)
            if (!aligned(p, 16)) return fail(DIT_ERR_ALIGN, "%s: image inputs must be 16-byte aligned", fn);
    }
    if (txt_rows > 0) {
        const void* ps[] = {txt_q, txt_k, txt_v, txt_q_w, txt_k_w, txt_cos, txt_sin};
        for (const void* p : ps)
            if (!aligned(p, 16)) return fail(DIT_ERR_ALIGN, "%s: text inputs must be 16-byte aligned", fn);
    }
    if (img_rows + txt_rows == 0) return ok();
    dit::QkvArgs a{};
    a.joint[0] = static_cast<uint16_t*>(joint_q);
    a.joint[1] = static_cast<uint16_t*>(joint_k);
    a.joint[2] = static_cast<uint16_t*>(joint_v);
    a.img[0] = static_cast<const uint16_t*>(img_q);
    a.img[1] = static_cast<const uint16_t*>(img_k);
    a.img[2] = static_cast<const uint16_t*>(img_v);
    a.txt[0] = static_cast<const uint16_t*>(txt_q);
    a.txt[1] = static_cast<const uint16_t*>(txt_k);
    a.txt[2] = static_cast<const uint16_t*>(txt_v);
    a.img_w[0] = static_cast<const uint16_t*>(img_q_w);
    a.img_w[1] = static_cast<const uint16_t*>(img_k_w);
    a.txt_w[0] = static_cast<const uint16_t*>(txt_q_w);
    a.txt_w[1] = static_cast<const uint16_t*>(txt_k_w);
    a.img_cos = img_cos;
    a.img_sin = img_sin;
    a.txt_cos = txt_cos;
    a.txt_sin = txt_sin;
    a.rope_stride = rope_row_stride;
    a.img_rows = img_rows;
    a.img_stride = img_row_stride;
    a.txt_rows = txt_rows;
    a.txt_stride = txt_row_stride;
    a.heads = heads;
    a.img_eps = img_eps;
    a.txt_eps = txt_eps;
    clear_stale_hip_error();
    return launched(dit::launch_qkv_epilogue(a, static_cast<hipStream_t>(stream)), fn);
}

int dit_bias_mul_add(void* y, const void* x, const void* bias, const void* gate,
                     const void* residual, int64_t rows, int64_t hidden, void* stream) {
    const char* fn = "dit_bias_mul_add";
    if (!y || !x || !gate || !residual) return fail(DIT_ERR_NULL, "%s: a required pointer is NULL", fn);
    if (rows < 0 || hidden <= 0)
        return fail(DIT_ERR_SHAPE, "%s: rows must be >= 0 and hidden > 0", fn);
    if (hidden % 8 != 0 || hidden > (int64_t(1) << 30))
        return fail(DIT_ERR_UNSUPPORTED, "%s: hidden (%lld) must be a multiple of 8 and <= 2^30", fn,
                    (long long)hidden);
    if (rows > kMaxRows) return fail(DIT_ERR_UNSUPPORTED, "%s: rows too large", fn);
    if (!aligned(y, 16) || !aligned(x, 16) || (bias && !aligned(bias, 16)) || !aligned(gate, 16) ||
        !aligned(residual, 16))
        return fail(DIT_ERR_ALIGN, "%s: tensors must be 16-byte aligned", fn);
    if (rows == 0) return ok();
    dit::BiasMulAddArgs a{};
    a.y = static_cast<uint16_t*>(y);
    a.x = static_cast<const uint16_t*>(x);
    a.bias = static_cast<const uint16_t*>(bias);
    a.gate = static_cast<const uint16_t*>(gate);
    a.residual = static_cast<const uint16_t*>(residual);
    a.rows = rows;
    a.hidden = hidden;
    clear_stale_hip_error();
    return launched(dit::launch_bias_mul_add(a, static_cast<hipStream_t>(stream)), fn);
}

int dit_token_cat_quant(int32_t kind, uint8_t* out, uint8_t* out_scales, const void* a,
                        int64_t a_cols, const void* b, int64_t b_cols, int64_t rows,
                        const float* scale_dev, void* stream) {
    const char* fn = "dit_token_cat_quant";
    if (kind != DIT_QUANT_FP8_E4M3 && kind != DIT_QUANT_FP4_E2M1 && kind != DIT_QUANT_FP4_E2M1_128X4)
        return fail(DIT_ERR_UNSUPPORTED, "%s: unknown quantisation kind %d", fn, kind);
    const bool fp4 = kind != DIT_QUANT_FP8_E4M3;
    if (rows < 0 || a_cols < 0 || b_cols < 0)
        return fail(DIT_ERR_SHAPE, "%s: sizes must be >= 0", fn);
    if (a_cols % 16 != 0 || b_cols % 16 != 0 || a_cols < 16)
        return fail(DIT_ERR_SHAPE, "%s: a_cols (%lld) and b_cols (%lld) must be multiples of 16, a_cols >= 16",
                    fn, (long long)a_cols, (long long)b_cols);
    if (a_cols > (int64_t(1) << 28) || b_cols > (int64_t(1) << 28) ||
        a_cols + b_cols > (int64_t(1) << 28) || rows > kMaxRows)
        return fail(DIT_ERR_UNSUPPORTED, "%s: shape too large", fn);
    if (kind == DIT_QUANT_FP4_E2M1_128X4 && (a_cols + b_cols) % 64 != 0)
        return fail(DIT_ERR_UNSUPPORTED, "%s: the 128x4 scale layout needs a_cols + b_cols %% 64 == 0",
                    fn);
    if (kind == DIT_QUANT_FP4_E2M1_128X4 && out_scales && !aligned(out_scales, 16))
        return fail(DIT_ERR_ALIGN, "%s: 128x4 scales must be 16-byte aligned", fn);
    if (!out || !a || !scale_dev || (b_cols > 0 && !b) ||
        (fp4 && !out_scales))
        return fail(DIT_ERR_NULL, "%s: a required pointer is NULL", fn);
    if (!aligned(out, 16) || !aligned(a, 16) || (b_cols > 0 && !aligned(b, 16)) ||
        !aligned(scale_dev, 4))
        return fail(DIT_ERR_ALIGN, "%s: tensors must be 16-byte aligned (scale 4-byte)", fn);
    if (rows == 0) return ok();
    dit::TokenCatArgs t{};
    t.out = out;
    t.out_scales = out_scales;
    t.a = static_cast<const uint16_t*>(a);
    t.b = static_cast<const uint16_t*>(b);
    t.a_cols = a_cols;
    t.b_cols = b_cols;
    t.rows = rows;
    t.scale = scale_dev;
    clear_stale_hip_error();
    const hipStream_t s = static_cast<hipStream_t>(stream);
    t.scales_tiled = kind == DIT_QUANT_FP4_E2M1_128X4;
    return launched(kind == DIT_QUANT_FP8_E4M3 ? dit::launch_token_cat_fp8(t, s)
                                               : dit::launch_token_cat_fp4(t, s),
                    fn);
}

}  // extern "C"

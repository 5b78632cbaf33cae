"""Fused DiT-block epilogues for MI355X (gfx950): HIP kernels behind a C ABI.

The entry points of include/dit_epilogues.h are exposed with the same names
(``dit_*``, raw pointers and sizes, caller-allocated outputs), plus allocating
conveniences that take and return torch device tensors:

  norm_modulate_fp8                 -> (y bf16, q e4m3 bytes)
  norm_modulate_fp8_dual            -> ((img_y, img_q), (txt_y, txt_q)), one launch
  scale_residual_norm_modulate_fp8  -> (residual_out, y, q)
  norm_modulate_fp4                 -> (y, FP4 packed bytes, scales)
  scale_residual_norm_modulate_fp4  -> (residual_out, y, FP4 packed bytes, scales)
  qkv_epilogue                      -> (joint_q, joint_k, joint_v)
  bias_mul_add                      -> y
  token_cat_quant                   -> FP8 bytes, or (FP4 packed bytes, scales)

The raw ``dit_*`` functions pass pointers through unchecked, as the C ABI
does; the conveniences check every tensor's dtype, shape and device first.
torch provides device memory and streams only; all arithmetic runs in the
library's kernels, and nothing falls back to the CPU.
"""
from __future__ import annotations

import torch

from ._native import (  # noqa: F401
    DIT_ERR_ALIGN, DIT_ERR_HIP, DIT_ERR_NULL, DIT_ERR_SHAPE, DIT_ERR_UNSUPPORTED, DIT_OK,
    DIT_FP4_SCALES_128X4, DIT_FP4_SCALES_ROW_MAJOR, DIT_QUANT_FP4_E2M1,
    DIT_QUANT_FP4_E2M1_128X4, DIT_QUANT_FP8_E4M3, LIB_PATH, DitError, dit_bias_mul_add,
    dit_norm_modulate_fp4, dit_norm_modulate_fp8, dit_norm_modulate_fp8_dual, dit_qkv_epilogue,
    dit_scale_residual_norm_modulate_fp4, dit_scale_residual_norm_modulate_fp8,
    dit_token_cat_quant, header_symbols, last_error, lib, status_string,
)


# Argument checks. The C ABI takes raw pointers and cannot see sizes, so these
# wrappers check every tensor against the sizes the kernels will read or write,
# and that all tensors sit on one GPU, before any pointer reaches a kernel.
# Shapes and dtypes are checked first, the device last.

def _bf16(t, name: str, shape=None) -> torch.Tensor:
    """A contiguous bf16 tensor, of `shape` if given."""
    if not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16:
        raise ValueError(f"{name} must be a bf16 tensor")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _scalar_f32(t, name: str) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or t.numel() != 1:
        raise ValueError(f"{name} must be a one-element fp32 tensor")
    return t


def _one_gpu(*tensors) -> None:
    """Every given tensor (None skipped) on one and the same GPU."""
    devs = {t.device for t in tensors if t is not None}
    if len(devs) != 1 or next(iter(devs)).type != "cuda":
        raise ValueError("all tensors must be on one GPU (one cuda device)")


def _rows_hidden(x, name: str = "x"):
    _bf16(x, name)
    if x.dim() < 1 or x.shape[-1] == 0:
        raise ValueError(f"{name} must have a non-empty last dimension")
    return x.numel() // x.shape[-1], x.shape[-1]


def _residual_args(x, bias, gate, residual, scale, shift, hidden) -> None:
    _bf16(residual, "residual", x.shape)
    for t, n in ((gate, "gate"), (scale, "scale"), (shift, "shift")):
        _bf16(t, n, (hidden,))
    if bias is not None:
        _bf16(bias, "bias", (hidden,))


def _outputs(x, want_y, want_q):
    if not (want_y or want_q):
        raise ValueError("at least one of the bf16 and FP8 outputs must be requested")
    y = torch.empty_like(x) if want_y else None
    q = torch.empty(x.shape, dtype=torch.uint8, device=x.device) if want_q else None
    return y, q


def norm_modulate_fp8(x: torch.Tensor, scale: torch.Tensor, shift: torch.Tensor,
                      input_scale: torch.Tensor | None, eps: float = 1e-6,
                      want_y: bool = True, want_q: bool = True):
    """LayerNorm (no affine) + AdaLN scale/shift + static FP8: returns (y, q);
    an output not asked for is None (and not written). x is [..., hidden];
    scale and shift are [hidden]; input_scale is a one-element fp32 tensor."""
    rows, hidden = _rows_hidden(x)
    _bf16(scale, "scale", (hidden,))
    _bf16(shift, "shift", (hidden,))
    s = _scalar_f32(input_scale, "input_scale") if want_q else None
    _one_gpu(x, scale, shift, s)
    y, q = _outputs(x, want_y, want_q)
    dit_norm_modulate_fp8(y, q, x, scale, shift, s, rows, hidden, eps)
    return y, q


def norm_modulate_fp8_dual(img_x, img_scale, img_shift, img_input_scale, txt_x, txt_scale,
                           txt_shift, txt_input_scale, img_eps: float = 1e-6,
                           txt_eps: float = 1e-6, want_y: bool = True, want_q: bool = True):
    """norm_modulate_fp8 on the image rows and the text rows of a block in one
    launch, each stream with its own modulation vectors, FP8 scale and eps:
    returns ((img_y, img_q), (txt_y, txt_q)). Both inputs share the hidden size."""
    img_rows, hidden = _rows_hidden(img_x, "img_x")
    txt_rows, txt_hidden = _rows_hidden(txt_x, "txt_x")
    if txt_hidden != hidden:
        raise ValueError(f"txt_x must have hidden {hidden}, got {txt_hidden}")
    for t, n in ((img_scale, "img_scale"), (img_shift, "img_shift"), (txt_scale, "txt_scale"),
                 (txt_shift, "txt_shift")):
        _bf16(t, n, (hidden,))
    si = _scalar_f32(img_input_scale, "img_input_scale") if want_q else None
    st = _scalar_f32(txt_input_scale, "txt_input_scale") if want_q else None
    _one_gpu(img_x, txt_x, img_scale, img_shift, txt_scale, txt_shift, si, st)
    yi, qi = _outputs(img_x, want_y, want_q)
    yt, qt = _outputs(txt_x, want_y, want_q)
    dit_norm_modulate_fp8_dual(yi, qi, img_x, img_scale, img_shift, si, img_rows, img_eps,
                               yt, qt, txt_x, txt_scale, txt_shift, st, txt_rows, txt_eps, hidden)
    return (yi, qi), (yt, qt)


def scale_residual_norm_modulate_fp8(x, bias, gate, residual, scale, shift, input_scale,
                                     eps: float = 1e-6, want_y: bool = True,
                                     want_q: bool = True):
    """bias (optional) + gated residual, then norm/modulate/FP8:
    returns (residual_out, y, q); an output not asked for is None. x and
    residual are [..., hidden]; bias, gate, scale and shift are [hidden]."""
    rows, hidden = _rows_hidden(x)
    _residual_args(x, bias, gate, residual, scale, shift, hidden)
    s = _scalar_f32(input_scale, "input_scale") if want_q else None
    _one_gpu(x, bias, gate, residual, scale, shift, s)
    r = torch.empty_like(x)
    y, q = _outputs(x, want_y, want_q)
    dit_scale_residual_norm_modulate_fp8(r, y, q, x, bias, gate, residual, scale, shift, s,
                                         rows, hidden, eps)
    return r, y, q


def _fp4_outputs(x, rows, hidden):
    packed = torch.empty((rows, hidden // 2), dtype=torch.uint8, device=x.device)
    scales = torch.empty(((rows + 127) // 128 * 128, hidden // 16), dtype=torch.uint8,
                         device=x.device)
    return packed, scales


def norm_modulate_fp4(x: torch.Tensor, scale: torch.Tensor, shift: torch.Tensor,
                      global_scale: torch.Tensor, eps: float = 1e-6, want_y: bool = True,
                      scale_layout: int = DIT_FP4_SCALES_ROW_MAJOR):
    """LayerNorm (no affine) + AdaLN scale/shift + 16-element-group FP4: returns
    (y or None, packed [rows, hidden/2], scales [round_up(rows,128), hidden/16])."""
    rows, hidden = _rows_hidden(x)
    _bf16(scale, "scale", (hidden,))
    _bf16(shift, "shift", (hidden,))
    _scalar_f32(global_scale, "global_scale")
    _one_gpu(x, scale, shift, global_scale)
    y = torch.empty_like(x) if want_y else None
    packed, scales = _fp4_outputs(x, rows, hidden)
    dit_norm_modulate_fp4(y, packed, scales, scale_layout, x, scale, shift, global_scale,
                          rows, hidden, eps)
    return y, packed, scales


def scale_residual_norm_modulate_fp4(x, bias, gate, residual, scale, shift, global_scale,
                                     eps: float = 1e-6, want_y: bool = True,
                                     scale_layout: int = DIT_FP4_SCALES_ROW_MAJOR):
    """bias (optional) + gated residual, then norm/modulate/FP4: returns
    (residual_out, y or None, packed, scales)."""
    rows, hidden = _rows_hidden(x)
    _residual_args(x, bias, gate, residual, scale, shift, hidden)
    _scalar_f32(global_scale, "global_scale")
    _one_gpu(x, bias, gate, residual, scale, shift, global_scale)
    r = torch.empty_like(x)
    y = torch.empty_like(x) if want_y else None
    packed, scales = _fp4_outputs(x, rows, hidden)
    dit_scale_residual_norm_modulate_fp4(r, y, packed, scales, scale_layout, x, bias, gate,
                                         residual, scale, shift, global_scale, rows, hidden,
                                         eps)
    return r, y, packed, scales


def _row_view(t, width: int, name: str) -> int:
    """Row stride (elements) of a [rows, width] bf16 view with unit column stride."""
    if not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16 or t.dim() != 2 \
            or t.shape[1] != width or t.stride(1) != 1:
        raise ValueError(f"{name} must be a [rows, {width}] bf16 view with unit column stride")
    return t.stride(0)


def qkv_epilogue(img_q, img_k, img_v, txt_q, txt_k, txt_v, img_q_w, img_k_w, txt_q_w,
                 txt_k_w, img_cos, img_sin, txt_cos, txt_sin, heads: int,
                 img_eps: float = 1e-6, txt_eps: float = 1e-6, head_dim: int = 128):
    """Q/K RMSNorm + interleaved RoPE + V copy into joint [text, image] buffers.
    img_*/txt_* are [rows, heads * head_dim] views (e.g. column slices of the
    packed QKV GEMM output). The four fp32 cos/sin tables are [rows, head_dim/2]
    views sharing one row stride (dense tables, or column halves of one
    [cos | sin] cache), with at least as many rows as their stream. Returns
    (joint_q, joint_k, joint_v), each [txt_rows + img_rows, heads, head_dim]."""
    width = heads * head_dim
    img_stride = _row_view(img_q, width, "img_q")
    txt_stride = _row_view(txt_q, width, "txt_q")
    n_img, n_txt = img_q.shape[0], txt_q.shape[0]
    for t, n, st, rows in ((img_k, "img_k", img_stride, n_img), (img_v, "img_v", img_stride, n_img),
                           (txt_k, "txt_k", txt_stride, n_txt), (txt_v, "txt_v", txt_stride, n_txt)):
        if _row_view(t, width, n) != st or t.shape[0] != rows:
            raise ValueError(f"{n} must have its stream's rows and row stride")
    for w, n in ((img_q_w, "img_q_w"), (img_k_w, "img_k_w"), (txt_q_w, "txt_q_w"),
                 (txt_k_w, "txt_k_w")):
        _bf16(w, n, (head_dim,))
    tables = [(t, n, rows) for t, n, rows in
              ((img_cos, "img_cos", n_img), (img_sin, "img_sin", n_img),
               (txt_cos, "txt_cos", n_txt), (txt_sin, "txt_sin", n_txt)) if rows]
    for t, n, rows in tables:
        if not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or t.dim() != 2 \
                or t.stride(1) != 1 or t.shape[1] != head_dim // 2:
            raise ValueError(f"{n} must be an fp32 [rows, head_dim/2] row view")
        if t.shape[0] < rows:
            raise ValueError(f"{n} has {t.shape[0]} rows, its stream has {rows}")
    rope_stride = tables[0][0].stride(0) if tables else head_dim // 2
    if any(t.stride(0) != rope_stride for t, _, _ in tables):
        raise ValueError("the cos/sin tables must share one row stride")
    _one_gpu(img_q, img_k, img_v, txt_q, txt_k, txt_v, img_q_w, img_k_w, txt_q_w, txt_k_w,
             *(t for t, _, _ in tables))
    out = [torch.empty((n_img + n_txt, heads, head_dim), dtype=torch.bfloat16,
                       device=img_q.device) for _ in range(3)]
    dit_qkv_epilogue(out[0], out[1], out[2], img_q, img_k, img_v, n_img, img_stride,
                     txt_q, txt_k, txt_v, n_txt, txt_stride, img_q_w, img_k_w,
                     txt_q_w, txt_k_w, img_cos, img_sin, txt_cos, txt_sin, rope_stride, heads,
                     head_dim, img_eps, txt_eps)
    return tuple(out)


def bias_mul_add(x, bias, gate, residual):
    """y = (x + bias) * gate + residual with one bf16 rounding of the multiply-add.
    x and residual are [..., hidden]; bias (optional) and gate are [hidden]."""
    rows, hidden = _rows_hidden(x)
    _bf16(residual, "residual", x.shape)
    _bf16(gate, "gate", (hidden,))
    if bias is not None:
        _bf16(bias, "bias", (hidden,))
    _one_gpu(x, bias, gate, residual)
    y = torch.empty_like(x)
    dit_bias_mul_add(y, x, bias, gate, residual, rows, hidden)
    return y


def token_cat_quant(kind: int, a: torch.Tensor, b: torch.Tensor | None,
                    scale: torch.Tensor):
    """Quantise the row concatenation [a | b] (a [rows, a_cols], b [rows, b_cols]
    or None). FP8: returns the E4M3 bytes [rows, cols]. FP4: returns (packed
    [rows, cols/2], scales [round_up(rows, 128), cols/16]); `scale` is then the
    global inverse scale. With DIT_QUANT_FP4_E2M1_128X4 the scales buffer holds
    the same bytes in the 128x4 tile layout."""
    _bf16(a, "a")
    if a.dim() != 2:
        raise ValueError("a must be [rows, a_cols]")
    rows, a_cols = a.shape
    if b is not None:
        _bf16(b, "b")
        if b.dim() != 2 or b.shape[0] != rows:
            raise ValueError(f"b must be [{rows}, b_cols], got {tuple(b.shape)}")
    _scalar_f32(scale, "scale")
    _one_gpu(a, b, scale)
    b_cols = 0 if b is None else b.shape[1]
    cols = a_cols + b_cols
    if kind == DIT_QUANT_FP8_E4M3:
        out = torch.empty((rows, cols), dtype=torch.uint8, device=a.device)
        dit_token_cat_quant(kind, out, None, a, a_cols, b, b_cols, rows, scale)
        return out
    packed = torch.empty((rows, cols // 2), dtype=torch.uint8, device=a.device)
    scales = torch.empty(((rows + 127) // 128 * 128, cols // 16), dtype=torch.uint8,
                         device=a.device)
    dit_token_cat_quant(kind, packed, scales, a, a_cols, b, b_cols, rows, scale)
    return packed, scales

"""ctypes binding of libdit_epilogues.so (the C ABI in include/dit_epilogues.h).

Argument marshalling only: tensors become device pointers, the stream defaults
to torch's current stream on the tensor's device, and a non-zero status
raises DitError. Every computation runs in the library's HIP kernels; there is
no CPU fallback. If the library is not built this module raises on first use.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libdit_epilogues.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "dit_epilogues.h")

DIT_OK = 0
DIT_ERR_NULL = 1
DIT_ERR_SHAPE = 2
DIT_ERR_ALIGN = 3
DIT_ERR_UNSUPPORTED = 4
DIT_ERR_HIP = 5
DIT_QUANT_FP8_E4M3 = 0
DIT_QUANT_FP4_E2M1 = 1
DIT_QUANT_FP4_E2M1_128X4 = 2
DIT_FP4_SCALES_ROW_MAJOR = 0
DIT_FP4_SCALES_128X4 = 1

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_F = ctypes.c_float

_SIGNATURES = {
    "dit_abi_version": (ctypes.c_int, []),
    "dit_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "dit_last_error": (ctypes.c_char_p, []),
    "dit_norm_modulate_fp8": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I64, _I64, _F, _P]),
    "dit_norm_modulate_fp8_dual":
        (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I64, _F, _P, _P, _P, _P, _P, _P, _I64, _F, _I64, _P]),
    "dit_scale_residual_norm_modulate_fp8":
        (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I64, _I64, _F, _P]),
    "dit_qkv_epilogue": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I64, _I64, _P, _P, _P, _I64,
                                        _I64, _P, _P, _P, _P, _P, _P, _P, _P, _I64, _I32, _I32,
                                        _F, _F, _P]),
    "dit_norm_modulate_fp4":
        (ctypes.c_int, [_P, _P, _P, _I32, _P, _P, _P, _P, _I64, _I64, _F, _P]),
    "dit_scale_residual_norm_modulate_fp4":
        (ctypes.c_int, [_P, _P, _P, _P, _I32, _P, _P, _P, _P, _P, _P, _P, _I64, _I64, _F, _P]),
    "dit_bias_mul_add": (ctypes.c_int, [_P, _P, _P, _P, _P, _I64, _I64, _P]),
    "dit_token_cat_quant": (ctypes.c_int, [_I32, _P, _P, _P, _I64, _P, _I64, _I64, _P, _P]),
}

_lib = None


class DitError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{status_string(status)}: {message}")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m quant_epilogues_amd._build` "
                "(there is no fallback implementation)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def header_symbols() -> list[str]:
    """Names of the functions include/dit_epilogues.h declares."""
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(dit_\w+)\s*\(", text, re.M)))


def status_string(status: int) -> str:
    return lib().dit_status_string(int(status)).decode()


def last_error() -> str:
    return lib().dit_last_error().decode()


def _check(status: int) -> None:
    if status != DIT_OK:
        raise DitError(status, last_error())


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("dit_epilogues takes device tensors")
    return t.data_ptr()


def _stream(stream, *tensors):
    if stream is not None:
        return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    for t in tensors:
        if isinstance(t, torch.Tensor):
            return torch.cuda.current_stream(t.device).cuda_stream
    return torch.cuda.current_stream().cuda_stream


# ---- entry points, same names and argument order as the C ABI -------------------

def dit_norm_modulate_fp8(y, q, x, scale, shift, input_scale_dev, rows, hidden, eps,
                          stream=None) -> None:
    _check(lib().dit_norm_modulate_fp8(_ptr(y), _ptr(q), _ptr(x), _ptr(scale), _ptr(shift),
                                       _ptr(input_scale_dev), rows, hidden, eps,
                                       _stream(stream, x)))


def dit_norm_modulate_fp8_dual(img_y, img_q, img_x, img_scale, img_shift, img_input_scale_dev,
                               img_rows, img_eps, txt_y, txt_q, txt_x, txt_scale, txt_shift,
                               txt_input_scale_dev, txt_rows, txt_eps, hidden, stream=None) -> None:
    _check(lib().dit_norm_modulate_fp8_dual(
        _ptr(img_y), _ptr(img_q), _ptr(img_x), _ptr(img_scale), _ptr(img_shift),
        _ptr(img_input_scale_dev), img_rows, img_eps, _ptr(txt_y), _ptr(txt_q), _ptr(txt_x),
        _ptr(txt_scale), _ptr(txt_shift), _ptr(txt_input_scale_dev), txt_rows, txt_eps, hidden,
        _stream(stream, img_x, txt_x)))


def dit_scale_residual_norm_modulate_fp8(residual_out, y, q, x, bias, gate, residual, scale,
                                         shift, input_scale_dev, rows, hidden, eps,
                                         stream=None) -> None:
    _check(lib().dit_scale_residual_norm_modulate_fp8(
        _ptr(residual_out), _ptr(y), _ptr(q), _ptr(x), _ptr(bias), _ptr(gate), _ptr(residual),
        _ptr(scale), _ptr(shift), _ptr(input_scale_dev), rows, hidden, eps, _stream(stream, x)))


def dit_qkv_epilogue(joint_q, joint_k, joint_v, img_q, img_k, img_v, img_rows, img_row_stride,
                     txt_q, txt_k, txt_v, txt_rows, txt_row_stride, img_q_w, img_k_w, txt_q_w,
                     txt_k_w, img_cos, img_sin, txt_cos, txt_sin, rope_row_stride, heads,
                     head_dim, img_eps, txt_eps, stream=None) -> None:
    _check(lib().dit_qkv_epilogue(
        _ptr(joint_q), _ptr(joint_k), _ptr(joint_v), _ptr(img_q), _ptr(img_k), _ptr(img_v),
        img_rows, img_row_stride, _ptr(txt_q), _ptr(txt_k), _ptr(txt_v), txt_rows,
        txt_row_stride, _ptr(img_q_w), _ptr(img_k_w), _ptr(txt_q_w), _ptr(txt_k_w),
        _ptr(img_cos), _ptr(img_sin), _ptr(txt_cos), _ptr(txt_sin), rope_row_stride, heads,
        head_dim, img_eps, txt_eps, _stream(stream, joint_q)))


def dit_norm_modulate_fp4(y, packed, scales, scale_layout, x, scale, shift, global_scale_dev,
                          rows, hidden, eps, stream=None) -> None:
    _check(lib().dit_norm_modulate_fp4(
        _ptr(y), _ptr(packed), _ptr(scales), scale_layout, _ptr(x), _ptr(scale), _ptr(shift),
        _ptr(global_scale_dev), rows, hidden, eps, _stream(stream, x)))


def dit_scale_residual_norm_modulate_fp4(residual_out, y, packed, scales, scale_layout, x, bias,
                                         gate, residual, scale, shift, global_scale_dev, rows,
                                         hidden, eps, stream=None) -> None:
    _check(lib().dit_scale_residual_norm_modulate_fp4(
        _ptr(residual_out), _ptr(y), _ptr(packed), _ptr(scales), scale_layout, _ptr(x),
        _ptr(bias), _ptr(gate), _ptr(residual), _ptr(scale), _ptr(shift), _ptr(global_scale_dev),
        rows, hidden, eps, _stream(stream, x)))


def dit_bias_mul_add(y, x, bias, gate, residual, rows, hidden, stream=None) -> None:
    _check(lib().dit_bias_mul_add(_ptr(y), _ptr(x), _ptr(bias), _ptr(gate), _ptr(residual),
                                  rows, hidden, _stream(stream, x)))


def dit_token_cat_quant(kind, out, out_scales, a, a_cols, b, b_cols, rows, scale_dev,
                        stream=None) -> None:
    _check(lib().dit_token_cat_quant(kind, _ptr(out), _ptr(out_scales), _ptr(a), a_cols,
                                     _ptr(b), b_cols, rows, _ptr(scale_dev),
                                     _stream(stream, a)))

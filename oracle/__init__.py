"""Python access to the plain CPU oracle (oracle.c) through ctypes.

TEST INFRASTRUCTURE. Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import this module. It never touches the
GPU library, and the GPU library never touches it.

Arrays are numpy arrays in host memory: bfloat16 tensors as uint16 bit
patterns, FP8 / packed FP4 as uint8, cos/sin tables as float32. Each function
allocates and returns its outputs.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_BUILT_PATH = os.path.join(_HERE, "liboracle.so")
# The library lib() loads. DIT_ORACLE_LIB points it at another build of
# oracle.c: the mutation tests load copies with planted mistakes this way to
# show that the pinning tests catch them.
_LIB_PATH = os.environ.get("DIT_ORACLE_LIB") or _BUILT_PATH

# Plain C, IEEE binary32/binary64, no FMA contraction, no fast-math.
CFLAGS = ["-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
          "-Wall", "-Wextra"]

_lib = None


def build(verbose: bool = False) -> str:
    """Compile oracle.c into liboracle.so next to it (always recompiles)."""
    return compile_source(_SRC, _BUILT_PATH, verbose)


def compile_source(src: str, out: str, verbose: bool = False) -> str:
    """Compile a copy of oracle.c (with oracle.h from this directory)."""
    cmd = ["gcc", *CFLAGS, f"-I{_HERE}", src, "-o", out, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return out


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        I32 = ctypes.c_int32
        F = ctypes.c_float
        D = ctypes.c_double
        sig = {
            "oracle_bf16_from_f32": (ctypes.c_uint16, [F]),
            "oracle_bf16_from_f64": (ctypes.c_uint16, [D]),
            "oracle_bf16_of_exact_sum": (ctypes.c_uint16, [D, D]),
            "oracle_f32_from_bf16": (F, [ctypes.c_uint16]),
            "oracle_e4m3_encode": (ctypes.c_uint8, [F]),
            "oracle_e4m3_decode": (D, [ctypes.c_uint8]),
            "oracle_e2m1_encode": (ctypes.c_uint8, [F]),
            "oracle_e2m1_decode": (D, [ctypes.c_uint8]),
            "oracle_bf16_from_f32_n": (None, [P, P, I64]),
            "oracle_bf16_from_f64_n": (None, [P, P, I64]),
            "oracle_bf16_of_exact_sum_n": (None, [P, P, P, I64]),
            "oracle_e4m3_encode_n": (None, [P, P, I64]),
            "oracle_e2m1_encode_n": (None, [P, P, I64]),
            "oracle_layernorm_stats": (None, [P, I64, F, P, P]),
            "oracle_rms_inverse": (F, [P, I64, F]),
            "oracle_norm_modulate_fp8": (None, [P, P, P, P, P, P, F, I64, I64, F]),
            "oracle_scale_residual_norm_modulate_fp8":
                (None, [P, P, P, P, P, P, P, P, P, P, F, I64, I64, F]),
            "oracle_qkv_epilogue": (None, [P, P, P, P, P, P, I64, I64, P, P, P, I64, I64,
                                           P, P, P, P, P, P, P, P, I32, I32, F, F]),
            "oracle_bias_mul_add": (None, [P, P, P, P, P, I64, I64]),
            "oracle_token_cat_fp8": (None, [P, P, P, I64, P, I64, I64, F]),
            "oracle_token_cat_fp4": (None, [P, P, P, P, P, I64, P, I64, I64, F]),
            "oracle_norm_modulate_fp4": (None, [P, P, P, P, P, P, P, P, F, I64, I64, F]),
            "oracle_fp4_scales_to_128x4": (None, [P, P, I64, I64]),
            "oracle_scale_residual_norm_modulate_fp4":
                (None, [P, P, P, P, P, P, P, P, P, P, P, P, F, I64, I64, F]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    assert a.dtype == np.uint16, a.dtype
    return a


# ---- codecs ------------------------------------------------------------------

def bf16_from_f32(v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, np.uint16)
    lib().oracle_bf16_from_f32_n(_ptr(v), _ptr(out), v.size)
    return out


def bf16_from_f64(v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(v.shape, np.uint16)
    lib().oracle_bf16_from_f64_n(_ptr(v), _ptr(out), v.size)
    return out


def bf16_of_exact_sum(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float64)
    b = np.ascontiguousarray(b, dtype=np.float64)
    out = np.empty(a.shape, np.uint16)
    lib().oracle_bf16_of_exact_sum_n(_ptr(a), _ptr(b), _ptr(out), a.size)
    return out


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, np.uint8)
    lib().oracle_e4m3_encode_n(_ptr(v), _ptr(out), v.size)
    return out


def e4m3_decode(codes) -> np.ndarray:
    L = lib()
    return np.array([L.oracle_e4m3_decode(int(c)) for c in np.asarray(codes).ravel()],
                    dtype=np.float64).reshape(np.shape(codes))


def e2m1_encode(v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, np.uint8)
    lib().oracle_e2m1_encode_n(_ptr(v), _ptr(out), v.size)
    return out


def e2m1_decode(codes) -> np.ndarray:
    L = lib()
    return np.array([L.oracle_e2m1_decode(int(c)) for c in np.asarray(codes).ravel()],
                    dtype=np.float64).reshape(np.shape(codes))


def f32_from_bf16(h: np.ndarray) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    return (h.astype(np.uint32) << 16).view(np.float32)


# ---- statistics ---------------------------------------------------------------

def layernorm_stats(v: np.ndarray, eps: float):
    v = _u16(v)
    m = ctypes.c_float()
    f = ctypes.c_float()
    lib().oracle_layernorm_stats(_ptr(v), v.size, eps, ctypes.byref(m), ctypes.byref(f))
    return np.float32(m.value), np.float32(f.value)


def rms_inverse(v: np.ndarray, eps: float) -> np.float32:
    v = _u16(v)
    return np.float32(lib().oracle_rms_inverse(_ptr(v), v.size, eps))


# ---- the five epilogues ----------------------------------------------------------

def norm_modulate_fp8(x, scale, shift, input_scale: float, eps: float):
    """Returns (y bf16 bits, q uint8, q_pre float32)."""
    x, scale, shift = _u16(x), _u16(scale), _u16(shift)
    rows, hidden = x.shape
    y = np.empty_like(x)
    q = np.empty(x.shape, np.uint8)
    pre = np.empty(x.shape, np.float32)
    lib().oracle_norm_modulate_fp8(_ptr(y), _ptr(q), _ptr(pre), _ptr(x), _ptr(scale),
                                   _ptr(shift), input_scale, rows, hidden, eps)
    return y, q, pre


def scale_residual_norm_modulate_fp8(x, bias, gate, residual, scale, shift,
                                     input_scale: float, eps: float):
    """Returns (residual_out bf16 bits, y bf16 bits, q uint8, q_pre float32)."""
    x, gate, residual, scale, shift = map(_u16, (x, gate, residual, scale, shift))
    bias = None if bias is None else _u16(bias)
    rows, hidden = x.shape
    r = np.empty_like(x)
    y = np.empty_like(x)
    q = np.empty(x.shape, np.uint8)
    pre = np.empty(x.shape, np.float32)
    lib().oracle_scale_residual_norm_modulate_fp8(
        _ptr(r), _ptr(y), _ptr(q), _ptr(pre), _ptr(x), _ptr(bias), _ptr(gate),
        _ptr(residual), _ptr(scale), _ptr(shift), input_scale, rows, hidden, eps)
    return r, y, q, pre


def qkv_epilogue(img_q, img_k, img_v, img_row_stride, txt_q, txt_k, txt_v, txt_row_stride,
                 img_rows, txt_rows, img_q_w, img_k_w, txt_q_w, txt_k_w,
                 img_cos, img_sin, txt_cos, txt_sin, heads, head_dim, img_eps, txt_eps):
    """img_*/txt_* are flat uint16 arrays whose row r, head h starts at
    r * row_stride + h * head_dim (pass the packed buffer offset to the Q/K/V
    column). Returns (joint_q, joint_k, joint_v) as [rows, heads, head_dim]."""
    n = txt_rows + img_rows
    jq = np.empty((n, heads, head_dim), np.uint16)
    jk = np.empty_like(jq)
    jv = np.empty_like(jq)
    f32 = lambda a: np.ascontiguousarray(a, dtype=np.float32)
    img_cos, img_sin, txt_cos, txt_sin = map(f32, (img_cos, img_sin, txt_cos, txt_sin))
    lib().oracle_qkv_epilogue(
        _ptr(jq), _ptr(jk), _ptr(jv), img_q, img_k, img_v, img_rows, img_row_stride,
        txt_q, txt_k, txt_v, txt_rows, txt_row_stride,
        _ptr(_u16(img_q_w)), _ptr(_u16(img_k_w)), _ptr(_u16(txt_q_w)), _ptr(_u16(txt_k_w)),
        _ptr(img_cos), _ptr(img_sin), _ptr(txt_cos), _ptr(txt_sin),
        heads, head_dim, img_eps, txt_eps)
    return jq, jk, jv


def qkv_epilogue_packed(img_qkv, txt_qkv, img_q_w, img_k_w, txt_q_w, txt_k_w,
                        img_cos, img_sin, txt_cos, txt_sin, heads, head_dim,
                        img_eps, txt_eps):
    """Convenience form for packed buffers [rows, 3 * heads * head_dim] whose
    Q, K, V are consecutive column blocks."""
    img_qkv, txt_qkv = _u16(img_qkv), _u16(txt_qkv)
    w = heads * head_dim
    ib, tb = img_qkv.ctypes.data, txt_qkv.ctypes.data
    return qkv_epilogue(ib, ib + 2 * w, ib + 4 * w, img_qkv.shape[1],
                        tb, tb + 2 * w, tb + 4 * w, txt_qkv.shape[1],
                        img_qkv.shape[0], txt_qkv.shape[0], img_q_w, img_k_w, txt_q_w,
                        txt_k_w, img_cos, img_sin, txt_cos, txt_sin, heads, head_dim,
                        img_eps, txt_eps)


def bias_mul_add(x, bias, gate, residual):
    x, gate, residual = map(_u16, (x, gate, residual))
    bias = None if bias is None else _u16(bias)
    rows, hidden = x.shape
    y = np.empty_like(x)
    lib().oracle_bias_mul_add(_ptr(y), _ptr(x), _ptr(bias), _ptr(gate), _ptr(residual),
                              rows, hidden)
    return y


def token_cat_fp8(a, b, input_scale: float):
    """Returns (q uint8 [rows, a_cols+b_cols], pre float32)."""
    a, b = _u16(a), _u16(b)
    rows = a.shape[0]
    cols = a.shape[1] + b.shape[1]
    out = np.empty((rows, cols), np.uint8)
    pre = np.empty((rows, cols), np.float32)
    lib().oracle_token_cat_fp8(_ptr(out), _ptr(pre), _ptr(a), a.shape[1], _ptr(b),
                               b.shape[1], rows, input_scale)
    return out, pre


def token_cat_fp4(a, b, g: float):
    """Returns (packed uint8 [rows, cols/2], scales uint8 [round_up(rows,128), cols/16],
    s_pre float32 [rows, cols/16], pre float32 [rows, cols])."""
    a, b = _u16(a), _u16(b)
    rows = a.shape[0]
    cols = a.shape[1] + b.shape[1]
    rows_pad = (rows + 127) // 128 * 128
    packed = np.empty((rows, cols // 2), np.uint8)
    scales = np.empty((rows_pad, cols // 16), np.uint8)
    s_pre = np.empty((rows, cols // 16), np.float32)
    pre = np.empty((rows, cols), np.float32)
    lib().oracle_token_cat_fp4(_ptr(packed), _ptr(scales), _ptr(s_pre), _ptr(pre), _ptr(a),
                               a.shape[1], _ptr(b), b.shape[1], rows, g)
    return packed, scales, s_pre, pre


def _fp4_outputs(rows, hidden):
    rows_pad = (rows + 127) // 128 * 128
    return (np.empty((rows, hidden // 2), np.uint8), np.empty((rows_pad, hidden // 16), np.uint8),
            np.empty((rows, hidden // 16), np.float32), np.empty((rows, hidden), np.float32))


def norm_modulate_fp4(x, scale, shift, g: float, eps: float):
    """LayerNorm + modulation, NVFP4 output. Returns (y bf16 bits, packed uint8
    [rows, hidden/2], scales uint8 [round_up(rows,128), hidden/16], s_pre, pre)."""
    x, scale, shift = _u16(x), _u16(scale), _u16(shift)
    rows, hidden = x.shape
    y = np.empty_like(x)
    packed, scales, s_pre, pre = _fp4_outputs(rows, hidden)
    lib().oracle_norm_modulate_fp4(_ptr(y), _ptr(packed), _ptr(scales), _ptr(s_pre), _ptr(pre),
                                   _ptr(x), _ptr(scale), _ptr(shift), g, rows, hidden, eps)
    return y, packed, scales, s_pre, pre


def scale_residual_norm_modulate_fp4(x, bias, gate, residual, scale, shift, g: float,
                                     eps: float):
    """bias + gated residual, LayerNorm + modulation, NVFP4 output. Returns
    (residual_out, y, packed, scales, s_pre, pre)."""
    x, gate, residual, scale, shift = map(_u16, (x, gate, residual, scale, shift))
    bias = None if bias is None else _u16(bias)
    rows, hidden = x.shape
    r = np.empty_like(x)
    y = np.empty_like(x)
    packed, scales, s_pre, pre = _fp4_outputs(rows, hidden)
    lib().oracle_scale_residual_norm_modulate_fp4(
        _ptr(r), _ptr(y), _ptr(packed), _ptr(scales), _ptr(s_pre), _ptr(pre), _ptr(x),
        _ptr(bias), _ptr(gate), _ptr(residual), _ptr(scale), _ptr(shift), g, rows, hidden, eps)
    return r, y, packed, scales, s_pre, pre


def fp4_scales_to_128x4(scales):
    """Row-major FP4 scales [rows_padded, groups] -> the 128x4 tile layout, as a
    flat uint8 array of the same size."""
    scales = np.ascontiguousarray(scales, np.uint8)
    rows_padded, groups = scales.shape
    assert rows_padded % 128 == 0 and groups % 4 == 0
    out = np.empty(scales.size, np.uint8)
    lib().oracle_fp4_scales_to_128x4(_ptr(out), _ptr(scales), rows_padded, groups)
    return out

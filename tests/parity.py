"""Tolerance checks for GPU-vs-oracle parity.

Rules (all outputs):
  * copies, packing and layout: bit-exact;
  * bf16: within 1 ulp on at least 99.99 % of elements and within 2 ulp on all
    (ulp distance = distance of the ordered bit patterns, +0 == -0);
  * FP8 / FP4 codes: a code may differ by one step only where the oracle's
    pre-rounding value lies within 1 bf16 ulp of the rounding boundary between
    the two codes (+0 == -0);
  * FP4 group scales: the same rule on the scale's pre-rounding value; for such
    a group the element codes are re-derived from the GPU's scale.
Each check returns the fraction of outputs that are bit-identical. With
exact=True it also requires every output to be bit-identical (after the
tolerance rule has been checked, so a failure says which bar was missed).
"""
from __future__ import annotations

import numpy as np

from exact import bf16_ulp_distance


def _bf16_ulp(v: np.ndarray) -> np.ndarray:
    a = np.abs(v.astype(np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0**-126)))
    return 2.0 ** (e - 7)


def _require_exact(name: str, gpu: np.ndarray, ref: np.ndarray, exact: bool) -> None:
    """exact=True: every output bit pattern equal (the sign of a zero included)."""
    if exact:
        n_diff = int(np.count_nonzero(gpu.reshape(-1) != ref.reshape(-1)))
        assert n_diff == 0, f"{name}: within tolerance but {n_diff} of {gpu.size} outputs differ"


def check_bf16(name: str, gpu: np.ndarray, ref: np.ndarray, exact: bool = False) -> float:
    assert gpu.shape == ref.shape, (name, gpu.shape, ref.shape)
    d = bf16_ulp_distance(gpu.reshape(-1), ref.reshape(-1))
    if d.size == 0:
        return 1.0
    worst = int(d.max())
    within1 = float((d <= 1).mean())
    assert worst <= 2, f"{name}: max bf16 distance {worst} ulp"
    assert within1 >= 0.9999, f"{name}: only {within1:.6f} within 1 ulp"
    _require_exact(name, gpu, ref, exact)
    return float((d == 0).mean())


def check_exact(name: str, gpu: np.ndarray, ref: np.ndarray) -> float:
    assert gpu.shape == ref.shape, (name, gpu.shape, ref.shape)
    bad = np.flatnonzero(gpu.reshape(-1) != ref.reshape(-1))
    assert bad.size == 0, f"{name}: {bad.size} bytes differ, first at {bad[:8]}"
    return 1.0


def _e4m3_key(c: np.ndarray) -> np.ndarray:
    c = c.astype(np.int64)
    return np.where(c < 0x80, c, -(c & 0x7F))


def _e4m3_value(c: np.ndarray, table: np.ndarray) -> np.ndarray:
    return table[c.astype(np.int64)]


def check_fp8(name: str, gpu: np.ndarray, ref: np.ndarray, pre: np.ndarray,
              e4m3_table: np.ndarray, exact: bool = False) -> float:
    """e4m3_table: value of each of the 256 codes (from the oracle's decoder)."""
    assert gpu.shape == ref.shape == pre.shape, name
    g, r, p = gpu.reshape(-1), ref.reshape(-1), pre.reshape(-1)
    kg, kr = _e4m3_key(g), _e4m3_key(r)
    diff = np.flatnonzero(kg != kr)
    if diff.size:
        assert np.all(np.abs(kg[diff] - kr[diff]) == 1), f"{name}: FP8 codes more than one step apart"
        boundary = 0.5 * (_e4m3_value(g[diff], e4m3_table) + _e4m3_value(r[diff], e4m3_table))
        near = np.abs(p[diff].astype(np.float64) - boundary) <= _bf16_ulp(p[diff])
        assert np.all(near), f"{name}: {int((~near).sum())} FP8 codes differ away from a boundary"
    _require_exact(name, gpu, ref, exact)
    return float(1.0 - diff.size / max(g.size, 1))


_E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _nibbles(packed: np.ndarray) -> np.ndarray:
    p = packed.astype(np.uint8)
    return np.stack([p & 0xF, p >> 4], axis=-1).reshape(p.shape[0], -1)


def _e2m1_key(n: np.ndarray) -> np.ndarray:
    n = n.astype(np.int64)
    return np.where(n & 8, -(n & 7), n & 7)


def _e2m1_value(n: np.ndarray) -> np.ndarray:
    n = n.astype(np.int64)
    return np.where(n & 8, -1.0, 1.0) * _E2M1[n & 7]


def check_fp4(name: str, gpu_packed, gpu_scales, ref_packed, ref_scales, s_pre, pre,
              x_f32: np.ndarray, g: float, e4m3_table: np.ndarray, e2m1_encode,
              exact: bool = False) -> tuple:
    """Returns (exact fraction of codes, exact fraction of scales). Codes are
    compared as values: +0 and -0 (0x0 and 0x8) are equal."""
    rows = ref_packed.shape[0]
    groups = ref_scales.shape[1]
    # Pad rows of the scale matrix must be exactly zero.
    check_exact(name + " pad scales", gpu_scales[rows:], ref_scales[rows:])
    gs, rs = gpu_scales[:rows].astype(np.int64), ref_scales[:rows].astype(np.int64)
    sdiff = gs != rs
    if sdiff.any():
        assert np.all(np.abs(gs[sdiff] - rs[sdiff]) == 1), f"{name}: scales more than one step apart"
        boundary = 0.5 * (e4m3_table[gs[sdiff]] + e4m3_table[rs[sdiff]])
        near = np.abs(s_pre[sdiff].astype(np.float64) - boundary) <= _bf16_ulp(s_pre[sdiff])
        assert np.all(near), f"{name}: {int((~near).sum())} group scales differ away from a boundary"
    ng, nr = _nibbles(gpu_packed), _nibbles(ref_packed)
    # For groups whose scale legitimately differs, re-derive the expected codes
    # from the GPU's scale with the oracle's encoder.
    exp_codes = nr.copy()
    exp_pre = pre.copy()
    if sdiff.any():
        for r_i, g_i in zip(*np.nonzero(sdiff)):
            sv = np.float32(e4m3_table[gs[r_i, g_i]])
            k = np.float32(np.float32(g) / sv) if sv != 0 else np.float32(0)
            xs = x_f32[r_i, 16 * g_i:16 * g_i + 16]
            t = (xs * k).astype(np.float32)
            codes = e2m1_encode(t) if sv != 0 else np.zeros(16, np.uint8)
            exp_codes[r_i, 16 * g_i:16 * g_i + 16] = codes
            exp_pre[r_i, 16 * g_i:16 * g_i + 16] = t
    kg, kr = _e2m1_key(ng), _e2m1_key(exp_codes)
    diff = kg != kr
    if diff.any():
        assert np.all(np.abs(kg[diff] - kr[diff]) == 1), f"{name}: FP4 codes more than one step apart"
        boundary = 0.5 * (_e2m1_value(ng[diff]) + _e2m1_value(exp_codes[diff]))
        p = exp_pre[diff].astype(np.float64)
        near = np.abs(np.abs(p) - np.abs(boundary)) <= _bf16_ulp(p)
        assert np.all(near), f"{name}: {int((~near).sum())} FP4 codes differ away from a boundary"
    _require_exact(name + " scales", gpu_scales[:rows], ref_scales[:rows], exact)
    _require_exact(name + " codes", np.asarray(gpu_packed), np.asarray(ref_packed), exact)
    return float(1.0 - diff.mean()), float(1.0 - sdiff.mean())

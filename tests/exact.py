"""Exact-rational helpers for pinning the oracle (CPU only).

Rounding here is done by brute force: list the representable neighbours of
a rational number and keep the nearest one, ties to the even bit pattern.
This shares nothing with oracle.c, which rounds by bit-spacing arithmetic.
"""
from __future__ import annotations

from decimal import Decimal, localcontext
from fractions import Fraction

import numpy as np


def _f32_from_bits(bits: int) -> float:
    return float(np.array([bits & 0xFFFFFFFF], np.uint32).view(np.float32)[0])


def bf16_value(bits: int) -> Fraction:
    return Fraction(_f32_from_bits((int(bits) & 0xFFFF) << 16))


def f32_value(x) -> Fraction:
    return Fraction(float(np.float32(x)))


def _key16(bits: int) -> int:
    return bits if bits < 0x8000 else -(bits & 0x7FFF)


def _bits16(key: int) -> int:
    return key if key >= 0 else (0x8000 | (-key))


def _key32(bits: int) -> int:
    return bits if bits < 0x80000000 else -(bits & 0x7FFFFFFF)


def _bits32(key: int) -> int:
    return key if key >= 0 else (0x80000000 | (-key))


def nearest_bf16_bits(x: Fraction) -> int:
    """Nearest finite bfloat16 to the rational x, ties to even pattern."""
    approx = np.float32(float(x))
    b32 = int(np.array([approx], np.float32).view(np.uint32)[0])
    k0 = _key16(b32 >> 16)
    best = None
    for k in range(k0 - 3, k0 + 4):
        bits = _bits16(k)
        if (bits & 0x7F80) == 0x7F80:  # inf / nan
            continue
        d = abs(bf16_value(bits) - x)
        cand = (d, bits & 1, bits)
        if best is None or cand < best:
            best = cand
    return best[2]


def nearest_f32(x: Fraction) -> np.float32:
    """Nearest finite binary32 to the rational x, ties to even pattern."""
    approx = np.float32(float(x))
    b0 = int(np.array([approx], np.float32).view(np.uint32)[0])
    k0 = _key32(b0)
    best = None
    for k in range(k0 - 3, k0 + 4):
        bits = _bits32(k)
        if (bits & 0x7F800000) == 0x7F800000:
            continue
        v = Fraction(_f32_from_bits(bits))
        cand = (abs(v - x), bits & 1, bits)
        if best is None or cand < best:
            best = cand
    return np.array([best[2]], np.uint32).view(np.float32)[0]


def bf16_ulp_distance(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Distance in representable steps between bf16 patterns (+0 == -0)."""
    a = a.astype(np.int64)
    b = b.astype(np.int64)
    ka = np.where(a < 0x8000, a, -(a & 0x7FFF))
    kb = np.where(b < 0x8000, b, -(b & 0x7FFF))
    return np.abs(ka - kb)


def is_bf16_midpoint(x: Fraction) -> bool:
    """True if x lies exactly halfway between two adjacent finite bfloat16 values."""
    k = _key16(nearest_bf16_bits(x))
    v = bf16_value(_bits16(k))
    for nb in (k - 1, k + 1):
        bits = _bits16(nb)
        if (bits & 0x7F80) == 0x7F80:
            continue
        if (v + bf16_value(bits)) / 2 == x:
            return True
    return False


def rsqrt_nearest_f32(t: Fraction) -> np.float32:
    """Nearest binary32 to 1 / sqrt(t) for a positive rational t. The root is
    taken with 80 significant decimal digits (decimal module), so the result
    is the correctly rounded one unless 1/sqrt(t) lies within 1e-79 (relative)
    of a binary32 midpoint."""
    with localcontext() as ctx:
        ctx.prec = 80
        r = Decimal(1) / (Decimal(t.numerator) / Decimal(t.denominator)).sqrt()
    return nearest_f32(Fraction(r))

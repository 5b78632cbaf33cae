"""Pins for the oracle's format codecs (CPU only).

bfloat16 and E4M3FN are checked against torch's CPU conversions (independent
library routines) and against brute-force exact rounding; E2M1 against the
tie table that follows from its eight magnitudes and against brute force.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from exact import bf16_value, nearest_bf16_bits

RNG = np.random.default_rng(1234)


def _torch_bf16_bits(v32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(v32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _all_finite_bf16() -> np.ndarray:
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    return bits[(bits & 0x7F80) != 0x7F80]


def test_bf16_from_f32_matches_torch(oracle_mod):
    raw = RNG.integers(0, 2**32, size=1_000_000, dtype=np.uint64).astype(np.uint32)
    # Ties and near-ties in the dropped half-word, both parities of the kept one.
    hi = RNG.integers(0, 2**16, size=20000, dtype=np.uint64).astype(np.uint32) << 16
    lows = np.array([0x8000, 0x7FFF, 0x8001, 0x0000, 0xFFFF], np.uint32)
    crafted = (hi[:, None] | lows[None, :]).ravel()
    bits = np.concatenate([raw, crafted])
    v = bits.view(np.float32)
    v = v[~np.isnan(v)]
    got = oracle_mod.bf16_from_f32(v)
    want = _torch_bf16_bits(v)
    assert np.array_equal(got, want)


def test_bf16_round_trip_is_identity_on_all_finite_patterns(oracle_mod):
    bits = _all_finite_bf16()
    v = oracle_mod.f32_from_bf16(bits)
    assert np.array_equal(oracle_mod.bf16_from_f32(v), bits)


def test_bf16_from_f64_matches_brute_force(oracle_mod):
    vals = list(RNG.standard_normal(300) * 10.0 ** RNG.integers(-6, 7, 300))
    # Doubles exactly on, and one binary64 step either side of, bf16 midpoints.
    for b in RNG.integers(0, 0x7F00, 200):
        mid = (bf16_value(int(b)) + bf16_value(int(b) + 1)) / 2
        m = float(mid)
        vals += [m, np.nextafter(m, np.inf), np.nextafter(m, -np.inf), -m]
    vals = np.array(vals, np.float64)
    got = oracle_mod.bf16_from_f64(vals)
    want = np.array([nearest_bf16_bits(Fraction(float(x))) for x in vals], np.uint16)
    assert np.array_equal(got, want)


def test_bf16_of_exact_sum_matches_brute_force(oracle_mod):
    def bf(n):
        return oracle_mod.f32_from_bf16(
            _torch_bf16_bits(RNG.standard_normal(n).astype(np.float32))).astype(np.float64)

    n = 2000
    a = bf(n) * bf(n) * 64.0  # a product of two bf16 values: exact in binary64
    b = bf(n)
    # Crafted: a exactly on a bf16 midpoint, b a tiny nudge of either sign or zero
    # (the double-rounding trap of a two-step fp32 evaluation).
    ca, cb = [], []
    for k in RNG.integers(0x3F00, 0x4A00, 300):
        mid = float((bf16_value(int(k)) + bf16_value(int(k) + 1)) / 2)
        # 2^-60 and 2^-100 sit beyond binary64's reach of the midpoint, so the
        # binary64 sum alone is a tie and only the TwoSum error breaks it.
        for nudge in (0.0, 2.0**-30, -(2.0**-30), 0.2080078125, -0.2080078125,
                      2.0**-60, -(2.0**-60), 2.0**-100, -(2.0**-100)):
            ca.append(mid)
            cb.append(nudge)
    a = np.concatenate([a, ca])
    b = np.concatenate([b, cb])
    got = oracle_mod.bf16_of_exact_sum(a, b)
    want = np.array([nearest_bf16_bits(Fraction(float(x)) + Fraction(float(y)))
                     for x, y in zip(a, b)], np.uint16)
    assert np.array_equal(got, want)


def test_e4m3_decode_matches_torch(oracle_mod):
    codes = np.arange(256, dtype=np.uint8)
    got = oracle_mod.e4m3_decode(codes)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])
    assert got[0x7E] == 448.0 and np.isnan(got[0x7F]) and np.isnan(got[0xFF])
    assert got[0x01] == 2.0**-9 and got[0x08] == 2.0**-6


# Scales used on the pages' paths: 1/0.0625, 1/0.02, 1/0.05, 1/0.5, identity, and
# the reciprocal of the midpoint-sensitive checkpoint scale the PR 37156 page names.
_INVS = [1.0, 16.0, 50.0, 20.0, 2.0, float(np.float32(1.0) / np.float32(0.4754464328))]


@pytest.mark.parametrize("inv", _INVS)
def test_e4m3_encode_matches_torch_on_all_bf16_products(oracle_mod, inv):
    bits = _all_finite_bf16()
    x = oracle_mod.f32_from_bf16(bits)
    with np.errstate(over="ignore"):
        v = np.clip(x * np.float32(inv), np.float32(-448.0), np.float32(448.0))
    v = v.astype(np.float32)
    got = oracle_mod.e4m3_encode(v)
    want = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, want)
    assert not np.any((got & 0x7F) == 0x7F)


def test_e4m3_encode_properties(oracle_mod):
    v = np.abs(RNG.standard_normal(200000).astype(np.float32)) * np.float32(100.0)
    v = np.concatenate([v, np.float32([0.0, 2.0**-10, 2.0**-9, 447.9, 448.0, 464.0, 1e6])])
    pos = oracle_mod.e4m3_encode(v)
    neg = oracle_mod.e4m3_encode(-v)
    assert np.array_equal(neg, pos | 0x80)  # symmetric, sign kept (also for zero)
    order = np.argsort(v, kind="stable")
    assert np.all(np.diff(pos[order].astype(np.int32)) >= 0)  # monotone
    assert oracle_mod.e4m3_encode(np.float32([448.0, 1e6]))[0] == 0x7E
    assert oracle_mod.e4m3_encode(np.float32([2.0**-10]))[0] == 0x00  # tie with 2^-9 -> even
    assert oracle_mod.e4m3_encode(np.float32([3 * 2.0**-10]))[0] == 0x02  # tie 1/2 -> even 2


def test_e2m1_encode_ties_and_grid(oracle_mod):
    grid = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    got = oracle_mod.e2m1_encode(np.float32(grid))
    assert list(got) == list(range(8))
    ties = {0.25: 0.0, 0.75: 1.0, 1.25: 1.0, 1.75: 2.0, 2.5: 2.0, 3.5: 4.0, 5.0: 4.0}
    codes = oracle_mod.e2m1_encode(np.float32(list(ties)))
    assert list(oracle_mod.e2m1_decode(codes)) == list(ties.values())
    assert list(oracle_mod.e2m1_encode(np.float32([6.5, 100.0, -7.0]))) == [7, 7, 15]
    assert list(oracle_mod.e2m1_encode(np.float32([-0.0, -0.1, -0.5]))) == [8, 8, 9]


def test_e2m1_encode_matches_brute_force(oracle_mod):
    grid = [Fraction(g) for g in (0, 0.5, 1, 1.5, 2, 3, 4, 6)]
    xs = [k / 64.0 for k in range(-480, 481)] + list(RNG.uniform(-8, 8, 2000))
    xs = np.array(xs, np.float32)
    got = oracle_mod.e2m1_encode(xs)
    for x, c in zip(xs, got):
        m = abs(Fraction(float(x)))
        best = min(range(8), key=lambda i: (abs(grid[i] - m), i & 1))
        if m > 6:
            best = 7
        assert c == (best | (8 if np.signbit(x) else 0)), (x, c, best)

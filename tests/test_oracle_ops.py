"""Pins for the oracle's five epilogues (CPU only).

Each function is checked against something other than itself: torch's CPU
layer_norm / rms_norm / bf16 add / fp8 conversion, exact rational arithmetic
(fractions, decimal), closed forms on constructed inputs, invariants, and the
tie case the sglang PR 37116 page gives for bias_mul_add.
"""
import json
import os
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import synth
from exact import (bf16_ulp_distance, bf16_value, is_bf16_midpoint, nearest_bf16_bits,
                   nearest_f32, rsqrt_nearest_f32)

RNG = np.random.default_rng(7)
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def bfbits(v) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf2f(bits) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def torch_e4m3(v32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(v32, np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


def rn32_inv(s: float) -> np.float32:
    return np.float32(1.0) / np.float32(s)


# ---------------------------------------------------------------------------
# LayerNorm + modulation + FP8
# ---------------------------------------------------------------------------

def _wide_row(rng, n):
    """bf16 values whose magnitudes span 2^-10 .. 2^20: a binary32 running sum
    of them is inexact, a binary64 one is exact (at most 47 significant bits)."""
    return rng.standard_normal(n) * 2.0 ** rng.integers(-10, 21, n)


@pytest.mark.parametrize("spread", ["normal", "wide"])
@pytest.mark.parametrize("n", [1, 2, 3, 5, 16, 32, 96])
def test_layernorm_stats_are_correctly_rounded(oracle_mod, n, spread):
    getcontext().prec = 80
    eps = np.float32(1e-6)
    rows = []
    for _ in range(10):
        if spread == "normal":
            rows.append(RNG.standard_normal(n) * 3.0 + RNG.standard_normal())
        else:
            rows.append(_wide_row(RNG, n))
    if spread == "wide" and n >= 3:
        # 2^24 + 1 is not a binary32 value: a binary32 sum drops the 1s.
        rows.append(np.array(([2.0**24, 1.0, -(2.0**24)] + [1.0] * n)[:n]))
    for row in rows:
        v = bfbits(row)
        xs = [bf16_value(b) for b in v]
        mean = sum(xs, Fraction(0)) / n
        var = sum(((x - mean) ** 2 for x in xs), Fraction(0)) / n
        t = var + Fraction(float(eps))
        inv = Decimal(1) / (Decimal(t.numerator) / Decimal(t.denominator)).sqrt()
        m, f = oracle_mod.layernorm_stats(v, float(eps))
        assert m == nearest_f32(mean)
        assert f == nearest_f32(Fraction(inv))


def test_norm_matches_torch_layer_norm(oracle_mod):
    # Rows at three magnitudes: eps matters for the smallest, not for the others.
    H = 3072
    x = np.concatenate([RNG.standard_normal((8, H)) * s for s in (1.0, 1e-3, 30.0)])
    xb = bfbits(x).reshape(x.shape)
    zeros = np.zeros(H, np.uint16)
    eps = float(np.float32(1e-6))
    y, _, _ = oracle_mod.norm_modulate_fp8(xb, zeros, zeros, 1.0, eps)
    ref = F.layer_norm(torch.from_numpy(bf2f(xb).astype(np.float64)), (H,), eps=eps)
    want = bfbits(ref.numpy().astype(np.float32))
    dist = bf16_ulp_distance(y, want)
    assert dist.max() <= 1
    assert (dist == 0).mean() >= 0.999


def test_norm_rows_have_zero_mean_unit_variance(oracle_mod):
    H = 3072
    for sigma in (0.5, 1.0, 4.0):
        x = bfbits(RNG.standard_normal((4, H)) * sigma + 0.3).reshape(4, H)
        zeros = np.zeros(H, np.uint16)
        y, _, _ = oracle_mod.norm_modulate_fp8(x, zeros, zeros, 1.0, 1e-6)
        yf = bf2f(y).astype(np.float64)
        xf = bf2f(x).astype(np.float64)
        var_x = xf.var(axis=1)
        assert np.all(np.abs(yf.mean(axis=1)) <= 2.0**-8)
        expect = var_x / (var_x + 1e-6)
        assert np.all(np.abs(yf.var(axis=1) - expect) <= 2.0**-7)


def test_norm_modulate_closed_form_alternating_rows(oracle_mod):
    # Rows +-1 alternating: mean 0, variance 1, so the normalised row is exactly
    # +-1 after bf16 rounding and y = sign * (1 + scale) + shift exactly.
    H = 512
    sign = np.where(np.arange(H) % 2 == 0, 1.0, -1.0)
    x = bfbits(np.stack([sign, -sign]))
    s_choices = np.array([-0.5, -0.25, 0.0, 0.125, 0.25, 0.5, 0.75])
    h_choices = np.array([-1.0, -0.375, 0.0, 0.25, 0.625])
    scale = RNG.choice(s_choices, H)
    shift = RNG.choice(h_choices, H)
    y, q, _ = oracle_mod.norm_modulate_fp8(x, bfbits(scale), bfbits(shift), 0.0625, 1e-6)
    want = np.stack([sign * (1 + scale) + shift, -sign * (1 + scale) + shift])
    assert np.array_equal(bf2f(y), want.astype(np.float32))
    assert np.array_equal(q, torch_e4m3(np.clip(want * 16.0, -448, 448)))


def test_constant_row_gives_shift(oracle_mod):
    H = 256
    x = bfbits(np.full((3, H), 2.5))
    scale = bfbits(RNG.standard_normal(H) * 0.1)
    shift = bfbits(RNG.standard_normal(H))
    y, q, _ = oracle_mod.norm_modulate_fp8(x, scale, shift, 0.02, 1e-6)
    assert np.array_equal(y, np.broadcast_to(shift, (3, H)))
    inv = rn32_inv(0.02)
    want_q = torch_e4m3(np.clip(bf2f(shift) * inv, -448, 448))
    assert np.array_equal(q, np.broadcast_to(want_q, (3, H)))


def _exact_norm_row(xbits, eps):
    """bf16 bits of one row's normalised values by reading c2, built from exact
    statistics: mean32 = RN32(mean) and factor32 = RN32(1 / sqrt(var + eps))
    from rationals (fractions, decimal), then RN32(RN32(v - mean32) * factor32)
    in numpy binary32 (IEEE), rounded to bf16 by torch."""
    xs = [bf16_value(b) for b in xbits]
    n = len(xs)
    mean = sum(xs, Fraction(0)) / n
    var = sum(((x - mean) ** 2 for x in xs), Fraction(0)) / n
    m32 = nearest_f32(mean)
    f32 = rsqrt_nearest_f32(var + Fraction(float(np.float32(eps))))
    return bfbits((bf2f(xbits) - m32) * f32)


def test_modulation_is_one_fused_multiply_add(oracle_mod):
    """y = bf16(RN32(norm * RN32(1 + scale) + shift)): the multiply-add is
    rounded once (reading c3: the page's single fp32 expression, which GPU
    compilers contract). Checked on every element against exact rationals.
    In row 0 every even column is constructed so that a product rounded to
    binary32 before the add gives a different y: scale = 3 * 2^-22, so that
    1 + scale carries bits far below the norm's own, and shift = -norm, so the
    exact result is the small norm * scale that a rounded product has lost."""
    H = 256
    rng = np.random.default_rng(31)
    x = bfbits(rng.standard_normal((2, H))).reshape(2, H)
    norm = np.stack([_exact_norm_row(x[r], 1e-6) for r in range(2)])
    scale = bfbits(rng.standard_normal(H) * 0.1)
    shift = bfbits(rng.standard_normal(H) * 0.1)
    cols = np.arange(0, H, 2)
    scale[cols] = bfbits(np.full(cols.size, 3 * 2.0**-22))
    shift[cols] = norm[0, cols] ^ 0x8000
    y, _, _ = oracle_mod.norm_modulate_fp8(x, scale, shift, 1.0, 1e-6)
    ops = np.float32(1.0) + bf2f(scale)  # RN32(1 + scale)
    want = np.array([[nearest_bf16_bits(Fraction(float(nearest_f32(
        bf16_value(norm[r, j]) * Fraction(float(ops[j])) + bf16_value(shift[j])))))
        for j in range(H)] for r in range(2)], np.uint16)
    assert np.array_equal(y, want)
    two_step = bfbits((bf2f(norm[0]) * ops) + bf2f(shift))  # product rounded first
    assert (two_step[cols] != want[0, cols]).mean() > 0.5


@pytest.mark.parametrize("input_scale", [0.02, 0.0625, 0.5, 0.4754464328])
def test_fp8_split_equals_fused(oracle_mod, input_scale):
    inp = synth.norm_modulate_inputs(rows=32, hidden=3072, seed=11, input_scale=input_scale)
    y, q, pre = oracle_mod.norm_modulate_fp8(
        synth.bf16_bits(inp.x), synth.bf16_bits(inp.scale), synth.bf16_bits(inp.shift),
        inp.input_scale, inp.eps)
    inv = rn32_inv(inp.input_scale)
    split = torch.from_numpy(bf2f(y)).mul(float(inv)).clamp(-448, 448)
    assert np.array_equal(q, split.to(torch.float8_e4m3fn).view(torch.uint8).numpy())
    assert np.array_equal(pre, split.numpy())
    assert not np.any((q & 0x7F) == 0x7F)


# ---------------------------------------------------------------------------
# Gated residual (+ optional bias)
# ---------------------------------------------------------------------------

def _tie_products(n_want: int):
    """(xb, gate) bf16 pairs whose exact product is a bf16 midpoint."""
    out = []
    while len(out) < n_want:
        a = bfbits(RNG.standard_normal(4096) * 4)
        g = bfbits(RNG.standard_normal(4096) * 4)
        for x, y in zip(a, g):
            if is_bf16_midpoint(bf16_value(x) * bf16_value(y)):
                out.append((x, y))
    return out[:n_want]


def test_gated_residual_is_one_exact_rounding(oracle_mod):
    H = 64
    rows = 6
    x = bfbits(RNG.standard_normal((rows, H))).reshape(rows, H)
    res = bfbits(RNG.standard_normal((rows, H))).reshape(rows, H)
    bias = bfbits(RNG.standard_normal(H) * 0.02)
    gate = bfbits(RNG.standard_normal(H) * 0.1 + 1)
    ties = _tie_products(H)
    # Row 0: the exact product lands on a bf16 midpoint; residual nudges it.
    nudges = bfbits(RNG.choice([1e-3, -1e-3, 0.0], H))
    x[0] = [t[0] for t in ties]
    gate_t = np.array([t[1] for t in ties], np.uint16)
    res[0] = nudges
    zeros = np.zeros(H, np.uint16)
    for g_row, bias_arg in ((gate, bias), (gate_t, None)):
        r_out, _, _, _ = oracle_mod.scale_residual_norm_modulate_fp8(
            x, bias_arg, g_row, res, zeros, zeros, 1.0, 1e-6)
        for i in range(rows):
            xb = bf2f(x[i])
            if bias_arg is not None:
                xb = bf2f(bfbits(xb + bf2f(bias_arg)))  # numpy fp32 add, torch bf16 RNE
            for j in range(H):
                exact = Fraction(float(bf2f(res[i, j]))) + Fraction(float(bf2f(g_row[j]))) * Fraction(float(xb[j]))
                assert r_out[i, j] == nearest_bf16_bits(exact), (i, j)


def _constructed_gated_columns(n_ties=24):
    """Columns (x, bias, gate, residual) of bf16 bits built so that each
    rounding rule of the gated multiply-add decides the result:
    - x = 1, bias = 2^-8 + 2^-10, gate = 3: rounding x + bias to bf16 first
      gives 3 * 1.0078125 = 3.0234375, a tie that goes to 3.03125; without
      that rounding the product is 3.017578125 -> 3.015625;
    - products exactly on a bf16 midpoint with residual +-2^-40 (or 0): an
      fp32 sum loses the residual and the tie goes to even, while the exact
      sum rounds toward the residual's sign;
    - the tie case printed on the sglang PR 37116 page."""
    ties = _tie_products(n_ties)
    cols = [(1.0, 2.0**-8 + 2.0**-10, 3.0, 0.0), (-1.0, -(2.0**-8 + 2.0**-10), 3.0, 0.0)]
    for k, (xt, gt) in enumerate(ties):
        nudge = (2.0**-40, -(2.0**-40), 0.0)[k % 3]
        cols.append((float(bf2f([xt])[0]), 0.0, float(bf2f([gt])[0]), nudge))
    with open(os.path.join(GOLDEN, "bias_mul_add_tie.json")) as f:
        case = json.load(f)["inputs"]
    cols.append((case["x"], case["bias"], case["gate"], case["residual"]))
    x, bias, gate, res = (bfbits([c[i] for c in cols]) for i in range(4))
    for i in range(4):  # every constructed value is a bf16 value
        assert np.array_equal(bf2f((x, bias, gate, res)[i]).astype(np.float64), [c[i] for c in cols])
    return x, bias, gate, res


def _gated_reference(x, bias, gate, res):
    """bf16(res + gate * bf16(RN32(x + bias))) with one exact final rounding."""
    xb = bf2f(bfbits(bf2f(x) + bf2f(bias)))  # numpy fp32 add, torch bf16 RNE
    return np.array([nearest_bf16_bits(bf16_value(r) + bf16_value(g) * Fraction(float(v)))
                     for v, g, r in zip(xb, gate, res)], np.uint16)


def test_gated_residual_constructed_rounding_cases(oracle_mod):
    x, bias, gate, res = _constructed_gated_columns()
    want = _gated_reference(x, bias, gate, res)
    assert bf2f(want[:2]).tolist() == [3.03125, -3.03125]
    zeros = np.zeros_like(x)
    r_out, _, _, _ = oracle_mod.scale_residual_norm_modulate_fp8(
        x.reshape(1, -1), bias, gate, res.reshape(1, -1), zeros, zeros, 1.0, 1e-6)
    assert np.array_equal(r_out[0], want)


def test_bias_mul_add_constructed_rounding_cases(oracle_mod):
    x, bias, gate, res = _constructed_gated_columns()
    want = _gated_reference(x, bias, gate, res)
    y = oracle_mod.bias_mul_add(x.reshape(1, -1), bias, gate, res.reshape(1, -1))
    assert np.array_equal(y[0], want)


def test_scale_residual_equals_norm_of_residual_out(oracle_mod):
    inp = synth.scale_residual_inputs(rows=24, hidden=3072, seed=5, input_scale=0.02)
    b = synth.bf16_bits
    r, y, q, pre = oracle_mod.scale_residual_norm_modulate_fp8(
        b(inp.x), b(inp.bias), b(inp.gate), b(inp.residual), b(inp.scale), b(inp.shift),
        inp.input_scale, inp.eps)
    y2, q2, pre2 = oracle_mod.norm_modulate_fp8(r, b(inp.scale), b(inp.shift), inp.input_scale,
                                                 inp.eps)
    assert np.array_equal(y, y2) and np.array_equal(q, q2) and np.array_equal(pre, pre2)
    # gate = 0: residual passes through untouched.
    zero_gate = np.zeros_like(b(inp.gate))
    r0, _, _, _ = oracle_mod.scale_residual_norm_modulate_fp8(
        b(inp.x), b(inp.bias), zero_gate, b(inp.residual), b(inp.scale), b(inp.shift),
        inp.input_scale, inp.eps)
    assert np.array_equal(r0, b(inp.residual))


# ---------------------------------------------------------------------------
# bias_mul_add
# ---------------------------------------------------------------------------

def test_bias_mul_add_golden_tie_case(oracle_mod):
    with open(os.path.join(GOLDEN, "bias_mul_add_tie.json")) as f:
        case = json.load(f)["inputs"]
    x, bias, gate, res = (bfbits([case[k]]) for k in ("x", "bias", "gate", "residual"))
    for k, v in zip(("x", "bias", "gate", "residual"), (x, bias, gate, res)):
        assert bf2f(v)[0] == np.float32(case[k]), k  # the page's inputs are bf16 values
    y = oracle_mod.bias_mul_add(x.reshape(1, 1), bias, gate, res.reshape(1, 1))
    biased = bf16_value(bfbits(bf2f(x) + bf2f(bias))[0])
    exact = biased * bf16_value(gate[0]) + bf16_value(res[0])
    want = nearest_bf16_bits(exact)
    assert y[0, 0] == want
    # The product alone is a bf16 midpoint: a two-step fp32 path rounds differently.
    two_step = bfbits(np.float32(biased * bf16_value(gate[0])) + bf2f(res))[0]
    assert two_step != want


def test_bias_mul_add_special_cases(oracle_mod):
    inp = synth.bias_mul_add_inputs(rows=16, hidden=512, seed=2)
    b = synth.bf16_bits
    y0 = oracle_mod.bias_mul_add(b(inp.x), b(inp.bias), np.zeros(512, np.uint16), b(inp.residual))
    assert np.array_equal(y0, b(inp.residual))
    one = bfbits(np.ones(512))
    y1 = oracle_mod.bias_mul_add(b(inp.x), None, one, b(inp.residual))
    assert np.array_equal(y1, b(inp.x + inp.residual))  # torch CPU bf16 add


def test_bias_mul_add_matches_exact_rationals(oracle_mod):
    rows, H = 4, 96
    inp = synth.bias_mul_add_inputs(rows=rows, hidden=H, seed=9)
    b = synth.bf16_bits
    x, bias, gate, res = b(inp.x), b(inp.bias), b(inp.gate), b(inp.residual)
    ties = _tie_products(H)  # (biased, gate) pairs on a midpoint; x chosen so bias keeps it
    x[0] = [t[0] for t in ties]
    bias = np.zeros(H, np.uint16)
    gate = np.array([t[1] for t in ties], np.uint16)
    res[0] = bfbits(RNG.choice([2.0**-20, -(2.0**-20), 0.0], H))
    y = oracle_mod.bias_mul_add(x, bias, gate, res)
    for i in range(rows):
        biased = bf2f(bfbits(bf2f(x[i]) + bf2f(bias)))
        for j in range(H):
            exact = Fraction(float(biased[j])) * bf16_value(gate[j]) + bf16_value(res[i, j])
            assert y[i, j] == nearest_bf16_bits(exact), (i, j)


# ---------------------------------------------------------------------------
# QKV epilogue
# ---------------------------------------------------------------------------

def _qkv_small(seed=0, img_rows=5, txt_rows=3, heads=3, img_eps=1e-6, txt_eps=0.25):
    return synth.qkv_inputs(img_rows=img_rows, txt_rows=txt_rows, heads=heads, head_dim=128,
                            seed=seed, img_eps=img_eps, txt_eps=txt_eps)


def _run_oracle_qkv(oracle_mod, inp, cos=None, sin=None):
    b = synth.bf16_bits
    ic, is_, tc, ts = inp.img_cos, inp.img_sin, inp.txt_cos, inp.txt_sin
    if cos is not None:
        ic, tc = np.full_like(ic, cos), np.full_like(tc, cos)
        is_, ts = np.full_like(is_, sin), np.full_like(ts, sin)
    return oracle_mod.qkv_epilogue_packed(
        b(inp.img_qkv), b(inp.txt_qkv), b(inp.img_q_w), b(inp.img_k_w), b(inp.txt_q_w),
        b(inp.txt_k_w), ic, is_, tc, ts, inp.heads, inp.head_dim, inp.img_eps, inp.txt_eps)


def test_qk_rmsnorm_matches_torch_rms_norm(oracle_mod):
    inp = _qkv_small()
    jq, jk, _ = _run_oracle_qkv(oracle_mod, inp, cos=1.0, sin=0.0)  # identity rotation
    D, Hh = inp.head_dim, inp.heads
    for part, out, (iw, tw) in ((0, jq, (inp.img_q_w, inp.txt_q_w)),
                                (1, jk, (inp.img_k_w, inp.txt_k_w))):
        for stream, w, eps, rows in (("txt", tw, inp.txt_eps, slice(0, 3)),
                                     ("img", iw, inp.img_eps, slice(3, 8))):
            t = (inp.txt_qkv if stream == "txt" else inp.img_qkv)
            x = t[:, part * Hh * D:(part + 1) * Hh * D].reshape(-1, Hh, D).double()
            ref = F.rms_norm(x, (D,), weight=w.double(), eps=float(np.float32(eps)))
            want = bfbits(ref.numpy().astype(np.float32)).reshape(-1, Hh, D)
            dist = bf16_ulp_distance(out[rows], want)
            assert dist.max() <= 1
            assert (dist == 0).mean() >= 0.998


def _head_mean_squares(heads_bits) -> list:
    """Exact mean of squares of each bf16 row (as Fractions), from integers:
    every bf16 value used here is a multiple of 2^-40 (checked)."""
    xi = bf2f(heads_bits).astype(np.float64) * 2.0**40
    assert np.all(xi == np.round(xi)) and np.all(np.abs(xi) < 2.0**62)
    xi = xi.astype(np.int64)
    d = heads_bits.shape[-1]
    return [Fraction(sum(int(v) * int(v) for v in row), d * 2**80) for row in xi]


def _exact_qk_norm(inp):
    """Joint [text, image] bf16 RMSNorm outputs of Q and K by reading c6, from
    exact statistics: inv = RN32(1 / sqrt(mean(x^2) + eps)) from rationals
    (fractions, decimal), then n = bf16(RN32(RN32(x * inv) * w)) with the two
    products in numpy binary32 (IEEE) and the bf16 rounding by torch."""
    b = synth.bf16_bits
    D, Hh, W = inp.head_dim, inp.heads, inp.width
    out = []
    for part in (0, 1):
        rows = []
        for stream in ("txt", "img"):
            packed = b(inp.txt_qkv if stream == "txt" else inp.img_qkv)
            w = bf2f(b(getattr(inp, f"{stream}_{'qk'[part]}_w")))
            eps = Fraction(float(np.float32(inp.txt_eps if stream == "txt" else inp.img_eps)))
            heads = packed[:, part * W:(part + 1) * W].reshape(-1, D)
            inv = np.array([rsqrt_nearest_f32(ms + eps) for ms in _head_mean_squares(heads)],
                           np.float32)
            rows.append(bfbits((bf2f(heads) * inv[:, None]) * w[None, :]).reshape(-1, Hh, D))
        out.append(np.concatenate(rows))
    return out


def _bf16_rne_bits(v32: np.ndarray) -> np.ndarray:
    """bf16 bits of finite binary32 values, round to nearest even (integer form,
    used only to pick constructed inputs)."""
    u = v32.view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def test_qk_rmsnorm_every_output_exact(oracle_mod):
    """Every Q/K output (identity rotation: cos 1, sin 0) equals
    bf16(RN32(RN32(x * inv) * w)) with the exactly rounded inv (reading c6).
    The two binary32 products of another order, x * (inv * w), differ from
    these by an ulp, which changes the bf16 output only near a bf16 midpoint;
    so columns of the image-Q weight are chosen, among the bf16 values in
    [1, 2), to put one image head's product on the other side of one."""
    inp = _qkv_small(seed=15, img_rows=512, txt_rows=4, heads=4)
    D, W = inp.head_dim, inp.width
    heads = synth.bf16_bits(inp.img_qkv)[:, :W].reshape(-1, D)  # every image-Q head
    eps = Fraction(float(np.float32(inp.img_eps)))
    invs = np.array([rsqrt_nearest_f32(ms + eps) for ms in _head_mean_squares(heads)], np.float32)
    cand = bf2f(np.arange(0x3F80, 0x4000, dtype=np.uint16))  # bf16 weights in [1, 2)
    w = synth.bf16_bits(inp.img_q_w).copy()
    built = 0
    for i in range(D):
        xs = bf2f(heads[:, i])
        ours = _bf16_rne_bits((xs * invs)[:, None] * cand[None, :])
        other = _bf16_rne_bits(xs[:, None] * (invs[:, None] * cand[None, :]))
        hit = np.flatnonzero((ours != other).any(axis=0))
        if hit.size:
            w[i] = bfbits(cand[hit[0]])[0]
            built += 1
    assert built >= D // 2
    inp.img_q_w = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16)
    jq, jk, _ = _run_oracle_qkv(oracle_mod, inp, cos=1.0, sin=0.0)
    nq, nk = _exact_qk_norm(inp)
    assert np.array_equal(jq, nq)
    assert np.array_equal(jk, nk)


@pytest.mark.parametrize("spread", ["normal", "wide"])
def test_rms_inverse_is_correctly_rounded(oracle_mod, spread):
    """RN32(1 / sqrt(mean(v^2) + eps)) against exact rationals and an
    80-digit root, over heads of 128 (and a few other lengths), at several
    magnitudes and epsilons (eps 0 included)."""
    rng = np.random.default_rng(21 if spread == "normal" else 22)
    for trial in range(160):
        n = 128 if trial % 4 else int(rng.integers(1, 130))
        v = rng.standard_normal(n)
        v = v * (10.0 ** rng.uniform(-3, 3) if spread == "normal" else 2.0 ** rng.integers(-30, 30, n))
        bits = bfbits(v)
        eps = float(np.float32((1e-6, 1e-5, 0.25, 0.0)[trial % 4]))
        ms = sum((bf16_value(b) ** 2 for b in bits), Fraction(0)) / n
        assert ms > 0
        assert oracle_mod.rms_inverse(bits, eps) == rsqrt_nearest_f32(ms + Fraction(eps)), trial


def _cos_on_bf16_midpoint(n0: Fraction, rng):
    """An fp32 c in [0.5, 1) for which RN32(n0 * c) is exactly a bf16 midpoint
    while n0 * c is not, and the exact product rounds to the other bf16
    neighbour than the tie rule picks for the midpoint; None if n0 is a power of
    two or zero (then n0 * c is exact in binary32)."""
    a = abs(n0)
    if a == 0 or (a.numerator & (a.numerator - 1) == 0 and a.denominator & (a.denominator - 1) == 0):
        return None
    for _ in range(400):
        p0 = a * Fraction(float(rng.uniform(0.5, 1.0)))
        lo = nearest_bf16_bits(p0)
        if bf16_value(lo) > p0:
            lo -= 1
        mid = (bf16_value(lo) + bf16_value(lo + 1)) / 2
        bits0 = int(np.array([mid / a], np.float32).view(np.uint32)[0])
        for k in range(-8, 9):  # fp32 values within 8 ulps of mid / n0
            c = np.array([bits0 + k], np.uint32).view(np.float32)[0]
            p = a * Fraction(float(c))
            if p != mid and Fraction(float(nearest_f32(p))) == mid and \
                    nearest_bf16_bits(p) != nearest_bf16_bits(mid) and 0.5 <= c < 1.0:
                return float(c)
    return None


def test_rope_every_output_exact(oracle_mod):
    """Every Q/K output of a small case equals the exact rotation
    (n0 c - n1 s, n1 c + n0 s) rounded once to bf16 (reading c7), where n is
    the RMSNorm output (the identity rotation gives it). Half of the cos/sin
    entries of Q head 0 are constructed (s = 0, c chosen so that RN32(n0 c)
    sits exactly on a bf16 midpoint that the exact product leaves on the other
    side): rounding each product to binary32 first gives another output there."""
    inp = _qkv_small(seed=16)
    nq, nk, _ = _run_oracle_qkv(oracle_mod, inp, cos=1.0, sin=0.0)
    n_txt = inp.txt_cos.shape[0]
    cos = np.concatenate([inp.txt_cos, inp.img_cos]).copy()
    sin = np.concatenate([inp.txt_sin, inp.img_sin]).copy()
    rng = np.random.default_rng(16)
    built = []
    for j in range(cos.shape[0]):
        for p in range(0, cos.shape[1], 2):
            c = _cos_on_bf16_midpoint(bf16_value(nq[j, 0, 2 * p]), rng)
            if c is not None:
                cos[j, p], sin[j, p] = c, 0.0
                built.append((j, p))
    assert len(built) >= cos.shape[0] * cos.shape[1] // 4
    inp.txt_cos, inp.img_cos = cos[:n_txt].copy(), cos[n_txt:].copy()
    inp.txt_sin, inp.img_sin = sin[:n_txt].copy(), sin[n_txt:].copy()
    oq, ok, _ = _run_oracle_qkv(oracle_mod, inp)
    for n, o in ((nq, oq), (nk, ok)):
        for j in range(o.shape[0]):
            for h in range(o.shape[1]):
                for p in range(cos.shape[1]):
                    n0, n1 = bf16_value(n[j, h, 2 * p]), bf16_value(n[j, h, 2 * p + 1])
                    c, s_ = Fraction(float(cos[j, p])), Fraction(float(sin[j, p]))
                    assert o[j, h, 2 * p] == nearest_bf16_bits(n0 * c - n1 * s_), (j, h, p)
                    assert o[j, h, 2 * p + 1] == nearest_bf16_bits(n1 * c + n0 * s_), (j, h, p)
    for j, p in built:  # a product rounded to binary32 first lands on the tie
        n0 = bf16_value(nq[j, 0, 2 * p])
        rounded = Fraction(float(nearest_f32(n0 * Fraction(float(cos[j, p])))))
        assert nearest_bf16_bits(rounded) != oq[j, 0, 2 * p]


def test_rope_is_complex_rotation_rounded_once(oracle_mod):
    inp = _qkv_small(seed=4)
    nq, nk, _ = _run_oracle_qkv(oracle_mod, inp, cos=1.0, sin=0.0)
    oq, ok, _ = _run_oracle_qkv(oracle_mod, inp)
    cos = np.concatenate([inp.txt_cos, inp.img_cos])  # joint order: text first
    sin = np.concatenate([inp.txt_sin, inp.img_sin])
    for n, o in ((nq, oq), (nk, ok)):
        nf = bf2f(n).astype(np.float64)
        z = (nf[..., 0::2] + 1j * nf[..., 1::2]) * (cos + 1j * sin)[:, None, :]
        want = np.empty_like(n)
        want[..., 0::2] = bfbits(z.real.astype(np.float32))
        want[..., 1::2] = bfbits(z.imag.astype(np.float32))
        dist = bf16_ulp_distance(o, want)
        assert dist.max() <= 1 and (dist == 0).mean() >= 0.998
        # Exactly: one rounding of the exact rotated value.
        for j in range(0, o.shape[0], 3):
            for h in range(o.shape[1]):
                for p in range(0, 64, 7):
                    n0 = Fraction(float(nf[j, h, 2 * p]))
                    n1 = Fraction(float(nf[j, h, 2 * p + 1]))
                    c = Fraction(float(cos[j, p]))
                    s = Fraction(float(sin[j, p]))
                    assert o[j, h, 2 * p] == nearest_bf16_bits(n0 * c - n1 * s)
                    assert o[j, h, 2 * p + 1] == nearest_bf16_bits(n1 * c + n0 * s)
        # The rotation preserves each pair's length (to bf16 rounding).
        of = bf2f(o).astype(np.float64)
        ln = np.hypot(nf[..., 0::2], nf[..., 1::2])
        lo = np.hypot(of[..., 0::2], of[..., 1::2])
        assert np.all(np.abs(lo - ln) <= 2.0**-7 * ln + 1e-30)


def test_qkv_layout_v_copy_and_joint_order(oracle_mod):
    inp = _qkv_small(seed=8)
    jq, jk, jv = _run_oracle_qkv(oracle_mod, inp)
    b = synth.bf16_bits
    w = inp.width
    tv = b(inp.txt_qkv)[:, 2 * w:].reshape(-1, inp.heads, inp.head_dim)
    iv = b(inp.img_qkv)[:, 2 * w:].reshape(-1, inp.heads, inp.head_dim)
    assert np.array_equal(jv[:3], tv) and np.array_equal(jv[3:], iv)
    # Contiguous inputs give the same result as the packed, strided views.
    tq, tk, tvv = (np.ascontiguousarray(b(x)) for x in inp.views("txt"))
    iq, ik, ivv = (np.ascontiguousarray(b(x)) for x in inp.views("img"))
    out = oracle_mod.qkv_epilogue(
        iq.ctypes.data, ik.ctypes.data, ivv.ctypes.data, w, tq.ctypes.data, tk.ctypes.data,
        tvv.ctypes.data, w, 5, 3, b(inp.img_q_w), b(inp.img_k_w), b(inp.txt_q_w),
        b(inp.txt_k_w), inp.img_cos, inp.img_sin, inp.txt_cos, inp.txt_sin, inp.heads,
        inp.head_dim, inp.img_eps, inp.txt_eps)
    for a, c in zip(out, (jq, jk, jv)):
        assert np.array_equal(a, c)


def test_qk_rmsnorm_unit_weight_gives_unit_rms(oracle_mod):
    inp = _qkv_small(seed=3, txt_eps=1e-6)
    one = torch.ones(128, dtype=torch.bfloat16)
    inp.img_q_w = inp.img_k_w = inp.txt_q_w = inp.txt_k_w = one
    jq, jk, _ = _run_oracle_qkv(oracle_mod, inp, cos=1.0, sin=0.0)
    for o in (jq, jk):
        rms = np.sqrt((bf2f(o).astype(np.float64) ** 2).mean(axis=-1))
        assert np.all(np.abs(rms - 1.0) <= 2.0**-8)


# ---------------------------------------------------------------------------
# Token concatenation + FP8 / FP4
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("input_scale", [0.05, 0.5, 0.4754464328])
def test_token_cat_fp8_equals_torch_cat_then_quantise(oracle_mod, input_scale):
    inp = synth.token_cat_inputs(rows=7, a_cols=96, b_cols=160, seed=1, fp8_scale=input_scale)
    b = synth.bf16_bits
    q, _ = oracle_mod.token_cat_fp8(b(inp.attn), b(inp.mlp), inp.fp8_scale)
    cat = torch.cat([inp.attn, inp.mlp], dim=1).float()
    ref = (cat * float(rn32_inv(inp.fp8_scale))).clamp(-448, 448).to(torch.float8_e4m3fn)
    assert np.array_equal(q, ref.view(torch.uint8).numpy())
    qa, _ = oracle_mod.token_cat_fp8(b(inp.attn), np.zeros((7, 0), np.uint16), inp.fp8_scale)
    qb, _ = oracle_mod.token_cat_fp8(b(inp.mlp), np.zeros((7, 0), np.uint16), inp.fp8_scale)
    assert np.array_equal(q, np.concatenate([qa, qb], axis=1))


_E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


@pytest.mark.parametrize("k,j", [(0, 0), (-3, 3), (2, -2), (-5, 6)])
def test_fp4_closed_form_grid_groups(oracle_mod, k, j):
    rows, a_cols, b_cols = 3, 32, 16
    cols = a_cols + b_cols
    idx = RNG.integers(0, 8, (rows, cols))
    neg = RNG.integers(0, 2, (rows, cols)).astype(bool)
    idx[:, ::16] = 7  # every group holds a +-6 * 2^k, so amax = 6 * 2^k
    vals = np.where(neg, -1.0, 1.0) * _E2M1[idx] * 2.0**k
    x = bfbits(vals).reshape(rows, cols)
    assert np.array_equal(bf2f(x), vals.astype(np.float32))
    g = 2.0**j
    packed, scales, s_pre, _ = oracle_mod.token_cat_fp4(x[:, :a_cols], x[:, a_cols:], g)
    # s_pre = (6 * 2^k / 6) * 2^j is exactly an E4M3 value; x * k_scale hits the grid.
    assert np.all(s_pre == np.float32(2.0 ** (k + j)))
    want_scale = torch_e4m3(np.float32([2.0 ** (k + j)]))[0]
    assert np.all(scales[:rows] == want_scale) and np.all(scales[rows:] == 0)
    codes = (idx | np.where(neg & (idx > 0), 8, 0)) | np.where(neg & (idx == 0), 8, 0)
    want_packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    assert np.array_equal(packed, want_packed)


def test_fp4_zero_group_saturation_and_padding(oracle_mod):
    rows, cols = 17, 64
    v = RNG.standard_normal((rows, cols))
    v[:, 16:32] = 0.0  # one all-zero group per row
    x = bfbits(v).reshape(rows, cols)
    packed, scales, _, _ = oracle_mod.token_cat_fp4(x[:, :32], x[:, 32:], 448.0 * 6 / 4.0)
    assert scales.shape == (128, 4)
    assert np.all(scales[:, 1] == 0) and np.all(packed[:, 8:16] == 0)
    assert np.all(scales[rows:] == 0)
    # Saturating global scale: every nonzero group's scale is 448, its largest element +-6.
    packed, scales, _, _ = oracle_mod.token_cat_fp4(x[:, :32], x[:, 32:], 1e4)
    big = np.abs(bf2f(x)).reshape(rows, 4, 16).max(axis=2) > 0.3
    assert np.all(scales[:rows][big] == 0x7E)
    nib = np.stack([packed & 0xF, packed >> 4], axis=-1).reshape(rows, cols)
    amax_pos = np.abs(bf2f(x)).reshape(rows, 4, 16).argmax(axis=2)
    for r in range(rows):
        for gi in range(4):
            if big[r, gi]:
                assert nib[r, gi * 16 + amax_pos[r, gi]] & 7 == 7


def test_fp4_dequantisation_error_bound_and_branch_split(oracle_mod):
    inp = synth.token_cat_inputs(rows=9, a_cols=64, b_cols=192, seed=6)
    b = synth.bf16_bits
    a_bits, m_bits = b(inp.attn), b(inp.mlp)
    packed, scales, s_pre, pre = oracle_mod.token_cat_fp4(a_bits, m_bits, inp.fp4_g)
    x = bf2f(np.concatenate([a_bits, m_bits], axis=1)).astype(np.float64)
    codes = np.stack([packed & 0xF, packed >> 4], axis=-1).reshape(x.shape)
    dec_s = oracle_mod.e4m3_decode(scales[:9]).repeat(16, axis=1)
    deq = oracle_mod.e2m1_decode(codes) * dec_s / inp.fp4_g
    kx = np.abs(x) * inp.fp4_g / dec_s
    half_gap = np.where(kx < 2, 0.25, np.where(kx < 4, 0.5, 1.0))
    ok = kx <= 6.0
    bound = half_gap * dec_s / inp.fp4_g * (1 + 2.0**-20)
    assert np.all(np.abs(x - deq)[ok] <= bound[ok])
    # An element can exceed 6 only when its group's E4M3 scale rounded down, which
    # is by at most 2^-4 relative, so it must lie within 2^-4 of the group maximum.
    amax = np.abs(x).reshape(9, -1, 16).max(axis=2).repeat(16, axis=1)
    assert np.all(np.abs(x)[~ok] >= amax[~ok] * (1 - 2.0**-4) * (1 - 2.0**-20))
    assert (~ok).mean() < 0.05
    # Groups never straddle the branch boundary: quantising each branch alone agrees.
    pa, sa, _, _ = oracle_mod.token_cat_fp4(a_bits, np.zeros((9, 0), np.uint16), inp.fp4_g)
    pb, sb, _, _ = oracle_mod.token_cat_fp4(m_bits, np.zeros((9, 0), np.uint16), inp.fp4_g)
    assert np.array_equal(packed, np.concatenate([pa, pb], axis=1))
    assert np.array_equal(scales, np.concatenate([sa, sb], axis=1))


def _fp4_reference(x_bits, g: float):
    """Group scale and element values by readings c10-c11, from rationals:
    s_pre = RN32(RN32(amax / 6) * g), s8 = e4m3(min(s_pre, 448)) by torch's
    conversion, pre = RN32(x * RN32(g / value(s8))) (0 where s8 is 0)."""
    xf = bf2f(x_bits).reshape(x_bits.shape[0], -1, 16)
    amax = np.abs(xf).max(axis=2)
    gq = Fraction(g)
    s_pre = np.array([[nearest_f32(Fraction(float(nearest_f32(Fraction(float(a)) / 6))) * gq)
                       for a in row] for row in amax], np.float32)
    s8 = torch_e4m3(np.minimum(s_pre, np.float32(448.0)))
    sval = torch.from_numpy(s8).view(torch.float8_e4m3fn).double().numpy()
    pre = np.zeros(xf.shape, np.float32)
    for r in range(xf.shape[0]):
        for gi in range(xf.shape[1]):
            if s8[r, gi] == 0:
                continue
            k = Fraction(float(nearest_f32(gq / Fraction(float(sval[r, gi])))))
            pre[r, gi] = [nearest_f32(Fraction(float(v)) * k) for v in xf[r, gi]]
    return s_pre, s8, pre.reshape(x_bits.shape)


@pytest.mark.parametrize("g", ["calibrated", 1.0, 3.7, 448.0, 0.01])
def test_fp4_group_arithmetic_exact(oracle_mod, g):
    """Every group's s_pre and scale byte and every element's pre-rounding
    value equal the rational reference of readings c10-c11, and every code is
    the E2M1 rounding of that value."""
    inp = synth.token_cat_inputs(rows=6, a_cols=64, b_cols=128, seed=17)
    b = synth.bf16_bits
    a_bits, m_bits = b(inp.attn), b(inp.mlp)
    gv = inp.fp4_g if g == "calibrated" else float(np.float32(g))
    packed, scales, s_pre, pre = oracle_mod.token_cat_fp4(a_bits, m_bits, gv)
    want_s_pre, want_s8, want_pre = _fp4_reference(np.concatenate([a_bits, m_bits], 1), gv)
    assert np.array_equal(s_pre, want_s_pre)
    assert np.array_equal(scales[:6], want_s8)
    assert np.array_equal(pre, want_pre)
    codes = np.stack([packed & 0xF, packed >> 4], axis=-1).reshape(6, -1)
    assert np.array_equal(codes, np.where(np.repeat(want_s8, 16, axis=1) == 0, 0,
                                          oracle_mod.e2m1_encode(want_pre)))


_E4M3_POS = torch.arange(0, 127, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()


def _scale_order_cases(n_want, rng):
    """(amax bf16 bits, g) with g close to 6 M / amax for an E4M3 midpoint M,
    kept where the scale byte of (amax / 6) * g differs from those of
    amax * (g / 6) and (amax * g) / 6 (binary32, used only to pick inputs)."""
    mids = (_E4M3_POS[21:-1] + _E4M3_POS[22:]) / 2
    out = []
    while len(out) < n_want:
        ab = int(rng.integers(0x3C00, 0x4200))
        amax = bf2f(np.array([ab], np.uint16))[0]
        g0 = int(np.array([rng.choice(mids) * 6 / float(amax)], np.float32).view(np.uint32)[0])
        for k in range(-4, 5):
            g = np.array([g0 + k], np.uint32).view(np.float32)[0]
            alt = [(amax / np.float32(6)) * g, amax * (g / np.float32(6)), (amax * g) / np.float32(6)]
            c = torch_e4m3(np.minimum(np.array(alt, np.float32), np.float32(448)))
            if c[0] != c[1] and c[0] != c[2]:
                out.append((ab, float(g)))
                break
    return out


def _element_order_cases(n_want, rng):
    """(x, amax bf16 bits, g) for which the E2M1 code of x * RN32(g / s) differs
    from that of RN32(x * g) / s, where s is the group's scale value: g is close
    to M s / x for an E2M1 midpoint M, and amax >= x gives scale s."""
    out = []
    while len(out) < n_want:
        x = bf2f(bfbits(np.array([rng.uniform(0.1, 4.0)])))[0]
        s8 = int(rng.integers(0x20, 0x70))
        sv = np.float32(_E4M3_POS[s8])
        m = float(rng.choice([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]))
        g0 = int(np.array([m * float(sv) / float(x)], np.float32).view(np.uint32)[0])
        for k in range(-3, 4):
            g = np.array([g0 + k], np.uint32).view(np.float32)[0]
            t1, t2 = x * (g / sv), (x * g) / sv
            e1, e2 = (_e2m1_index_brute(t) for t in (t1, t2))
            if e1 == e2:
                continue
            a0 = int(bfbits(np.array([6 * float(sv) / float(g)]))[0])
            for ab in range(a0 - 3, a0 + 4):
                amax = bf2f(np.array([ab], np.uint16))[0]
                if amax >= x and torch_e4m3(np.array([min((amax / np.float32(6)) * g, 448)],
                                                     np.float32))[0] == s8:
                    out.append((int(bfbits(np.array([x]))[0]), ab, float(g)))
                    break
            break
    return out


def _e2m1_index_brute(t: float) -> int:
    """E2M1 magnitude index of t by brute force over the grid, ties to the even
    index (used only to pick inputs)."""
    d = np.abs(np.abs(t) - _E2M1)
    best = np.flatnonzero(d == d.min())
    return int(best[0] if best.size == 1 or best[0] % 2 == 0 else best[1])


def test_fp4_rounding_orders_constructed(oracle_mod):
    """Groups built so that the other orders of the scale arithmetic (amax * g
    / 6, amax * (g / 6)) give another scale byte, and of the element arithmetic
    ((x * g) / s) another code, than the reading's order: the oracle matches the
    rational reference of readings c10-c11 on each."""
    rng = np.random.default_rng(41)
    for ab, g in _scale_order_cases(8, rng):
        row = np.zeros((1, 16), np.uint16)
        row[0, 0] = ab
        row[0, 5] = ab ^ 0x8000 if ab > 0x3C80 else 0x3C00
        packed, scales, s_pre, pre = oracle_mod.token_cat_fp4(row, np.zeros((1, 0), np.uint16), g)
        ws, w8, wp = _fp4_reference(row, g)
        assert s_pre[0, 0] == ws[0, 0] and scales[0, 0] == w8[0, 0] and np.array_equal(pre, wp)
    for xb, ab, g in _element_order_cases(8, rng):
        row = np.zeros((1, 16), np.uint16)
        row[0, 0], row[0, 3] = ab, xb
        packed, scales, s_pre, pre = oracle_mod.token_cat_fp4(row, np.zeros((1, 0), np.uint16), g)
        ws, w8, wp = _fp4_reference(row, g)
        assert scales[0, 0] == w8[0, 0] and np.array_equal(pre, wp)
        code3 = (packed[0, 1] >> 4) & 7
        assert code3 == _e2m1_index_brute(float(wp[0, 3]))


# ---------------------------------------------------------------------------
# NVFP4 output on the LayerNorm path
# ---------------------------------------------------------------------------

def test_norm_fp4_closed_form_alternating_rows(oracle_mod):
    """Rows alternating +a, -a (a >= 1) normalise to exactly +-1, so with scale =
    shift = 0 and g = 6 every group has amax 1, s_pre = 1 (scale code 0x38),
    element scale 6 and codes +-6: each byte is 0xF7 (+6 low, -6 high)."""
    rows, hidden = 5, 256
    a = np.array([1.0, 1.5, 2.0, 3.0, 96.0], np.float32)
    x = np.tile(np.array([1.0, -1.0], np.float32), hidden // 2)[None, :] * a[:, None]
    zeros = np.zeros(hidden, np.uint16)
    y, packed, scales, s_pre, _ = oracle_mod.norm_modulate_fp4(bfbits(x).reshape(rows, hidden),
                                                               zeros, zeros, 6.0, 1e-6)
    assert np.array_equal(bf2f(y).reshape(rows, hidden), np.sign(x))
    assert np.all(packed == 0xF7)
    assert np.all(s_pre == 1.0) and np.all(scales[:rows] == 0x38) and np.all(scales[rows:] == 0)


@pytest.mark.parametrize("g", [1.0, 448.0, 1e4])
def test_norm_fp4_is_the_fp4_of_the_bf16_y(oracle_mod, g):
    """Fused == split: y equals the FP8 variant's y, and the NVFP4 outputs equal
    the token-cat FP4 quantiser applied to that y."""
    inp = synth.norm_modulate_inputs(rows=9, hidden=512, seed=12)
    b = synth.bf16_bits
    y, packed, scales, s_pre, pre = oracle_mod.norm_modulate_fp4(
        b(inp.x), b(inp.scale), b(inp.shift), g, inp.eps)
    y8, _, _ = oracle_mod.norm_modulate_fp8(b(inp.x), b(inp.scale), b(inp.shift), 0.0625, inp.eps)
    assert np.array_equal(y, y8)
    p2, s2, sp2, pre2 = oracle_mod.token_cat_fp4(y, np.zeros((9, 0), np.uint16), g)
    assert np.array_equal(packed, p2) and np.array_equal(scales, s2)
    assert np.array_equal(s_pre, sp2) and np.array_equal(pre, pre2)


def test_scale_residual_fp4_is_the_norm_fp4_of_residual_out(oracle_mod):
    inp = synth.scale_residual_inputs(rows=7, hidden=1024, seed=13)
    b = synth.bf16_bits
    r, y, packed, scales, _, _ = oracle_mod.scale_residual_norm_modulate_fp4(
        b(inp.x), b(inp.bias), b(inp.gate), b(inp.residual), b(inp.scale), b(inp.shift), 448.0,
        inp.eps)
    r8, _, _, _ = oracle_mod.scale_residual_norm_modulate_fp8(
        b(inp.x), b(inp.bias), b(inp.gate), b(inp.residual), b(inp.scale), b(inp.shift), 0.0625,
        inp.eps)
    assert np.array_equal(r, r8)
    y2, p2, s2, _, _ = oracle_mod.norm_modulate_fp4(r, b(inp.scale), b(inp.shift), 448.0, inp.eps)
    assert np.array_equal(y, y2) and np.array_equal(packed, p2) and np.array_equal(scales, s2)


# ---------------------------------------------------------------------------
# 128x4 FP4 scale layout
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("rows_padded,groups", [(128, 4), (256, 12), (384, 1536 // 16)])
def test_fp4_scale_layout_matches_tensor_reshape(oracle_mod, rows_padded, groups):
    """The layout as a tensor view: [Mt, 128, Kt, 4] -> split the 128 rows as
    (4, 32) -> order (Mt, Kt, 32, 4, 4). Every byte is a distinct tag, so the
    comparison checks the whole permutation."""
    tags = np.arange(rows_padded * groups, dtype=np.int64)
    s = (tags % 251).astype(np.uint8).reshape(rows_padded, groups)  # byte tags
    want_idx = (tags.reshape(rows_padded // 128, 4, 32, groups // 4, 4)
                .transpose(0, 3, 2, 1, 4).reshape(-1))
    got = oracle_mod.fp4_scales_to_128x4(s)
    assert np.array_equal(got, s.reshape(-1)[want_idx])


def test_fp4_scale_layout_tiles_are_contiguous_and_complete(oracle_mod):
    """Each 128 x 4 block of the matrix lands in one 512-byte range, blocks
    in row-major block order, and every byte appears once."""
    rows_padded, groups = 256, 8
    ids = np.arange(rows_padded * groups, dtype=np.int64)
    lo = oracle_mod.fp4_scales_to_128x4((ids & 0xFF).astype(np.uint8).reshape(rows_padded, groups))
    hi = oracle_mod.fp4_scales_to_128x4((ids >> 8).astype(np.uint8).reshape(rows_padded, groups))
    back = lo.astype(np.int64) | (hi.astype(np.int64) << 8)
    assert np.array_equal(np.sort(back), ids)
    m, k = back // groups, back % groups
    tile = (m // 128) * (groups // 4) + k // 4
    assert np.array_equal(tile, np.arange(back.size) // 512)
    # Inside a tile: the first 16 bytes are rows 0, 32, 64, 96, four scales each.
    assert list(m[:16]) == [0] * 4 + [32] * 4 + [64] * 4 + [96] * 4
    assert list(k[:16]) == [0, 1, 2, 3] * 4

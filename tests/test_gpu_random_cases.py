"""GPU parity on randomly drawn shapes, scales and value ranges.

The cases are drawn once from fixed seeds (so every run checks the same
cases). They vary what the fixed cases hold still: row and head counts, widths
(any multiple of 8 or 16 up to the limits), FP8 and FP4 scales over several
decades, epsilons, per-row magnitudes over eight decades, rows with a
common offset (a mean several spreads away from zero) and rows with many
exact zeros.
Every output must equal the oracle's byte for byte, as in the fixed cases.
"""
import numpy as np
import pytest
import torch

import synth
from parity import check_exact
from test_gpu_parity import (Guarded, _oracle_qkv, _print_case, _run_qkv, bits, check_bf16,
                             check_fp4, check_fp8, dev, dscalar, e4m3_table, qe)  # noqa: F401

pytestmark = pytest.mark.gpu

N_CASES = 24


def _rows_bf16(g: torch.Generator, rows: int, cols: int) -> torch.Tensor:
    """Rows of N(0,1) values, each row scaled by 10^U(-4,4); a fifth of the
    rows get a common offset of up to 8 spreads, a fifth lose about half of
    their values to exact zeros."""
    x = torch.randn(rows, cols, generator=g, dtype=torch.float32)
    u = torch.rand(rows, 3, generator=g, dtype=torch.float32)
    off = torch.where(u[:, :1] < 0.2, 8.0 * (2.0 * u[:, 1:2] - 1.0), torch.zeros(rows, 1))
    x = x + off
    drop = (u[:, 2:3] < 0.2) & (torch.rand(rows, cols, generator=g) < 0.5)
    x = torch.where(drop, torch.zeros(()), x)
    mag = 10.0 ** (8.0 * torch.rand(rows, 1, generator=g) - 4.0)
    return (x * mag).to(torch.bfloat16)


def _vec(g: torch.Generator, n: int, mean: float, std: float) -> torch.Tensor:
    return (torch.randn(n, generator=g) * std + mean).to(torch.bfloat16)


def _log_uniform(rng, lo, hi) -> float:
    return float(np.float32(10.0 ** rng.uniform(np.log10(lo), np.log10(hi))))


def _norm_case(i):
    rng = np.random.default_rng(1000 + i)
    hidden = 8 * int(rng.integers(1, 1025))
    rows = int(rng.integers(1, max(2, min(1500, 3_000_000 // hidden))))
    return dict(rows=rows, hidden=hidden, input_scale=_log_uniform(rng, 1e-3, 1e2),
                eps=float(rng.choice([1e-6, 1e-5, 1e-3])), resid=bool(rng.integers(0, 2)),
                with_bias=bool(rng.integers(0, 2)), seed=2000 + i)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_norm_fp8(qe, oracle_mod, e4m3_table, i):
    c = _norm_case(i)
    _print_case("random norm fp8", c)
    rows, hidden = c["rows"], c["hidden"]
    g = torch.Generator().manual_seed(c["seed"])
    x = _rows_bf16(g, rows, hidden)
    scale, shift = _vec(g, hidden, 0.0, 0.3), _vec(g, hidden, 0.0, 0.3)
    y = Guarded((rows, hidden), torch.bfloat16)
    q = Guarded((rows, hidden), torch.uint8)
    if c["resid"]:
        residual = _rows_bf16(g, rows, hidden)
        gate = _vec(g, hidden, 1.0, 0.5)
        bias = _vec(g, hidden, 0.0, 0.05) if c["with_bias"] else None
        r = Guarded((rows, hidden), torch.bfloat16)
        qe.dit_scale_residual_norm_modulate_fp8(
            r.t, y.t, q.t, dev(x), dev(bias), dev(gate), dev(residual), dev(scale), dev(shift),
            dscalar(c["input_scale"]), rows, hidden, c["eps"])
        rr, ry, rq, pre = oracle_mod.scale_residual_norm_modulate_fp8(
            bits(x), None if bias is None else bits(bias), bits(gate), bits(residual),
            bits(scale), bits(shift), c["input_scale"], c["eps"])
        torch.cuda.synchronize()
        r.check("r")
        check_bf16("residual_out", r.bits(), rr)
    else:
        qe.dit_norm_modulate_fp8(y.t, q.t, dev(x), dev(scale), dev(shift),
                                 dscalar(c["input_scale"]), rows, hidden, c["eps"])
        ry, rq, pre = oracle_mod.norm_modulate_fp8(bits(x), bits(scale), bits(shift),
                                                   c["input_scale"], c["eps"])
        torch.cuda.synchronize()
    y.check("y"), q.check("q")
    check_bf16("y", y.bits(), ry)
    check_fp8("q", q.bits(), rq, pre, e4m3_table)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_norm_fp4(qe, oracle_mod, e4m3_table, i):
    c = _norm_case(100 + i)
    hidden = (c["hidden"] + 15) // 16 * 16
    rows = c["rows"]
    rng = np.random.default_rng(3000 + i)
    gv = _log_uniform(rng, 1e-2, 1e4)
    tiled = hidden % 64 == 0 and bool(rng.integers(0, 2))
    _print_case("random norm fp4", c, hidden, gv, tiled)
    layout = qe.DIT_FP4_SCALES_128X4 if tiled else qe.DIT_FP4_SCALES_ROW_MAJOR
    g = torch.Generator().manual_seed(c["seed"])
    x = _rows_bf16(g, rows, hidden)
    scale, shift = _vec(g, hidden, 0.0, 0.3), _vec(g, hidden, 0.0, 0.3)
    rows_pad = (rows + 127) // 128 * 128
    y = Guarded((rows, hidden), torch.bfloat16)
    packed = Guarded((rows, hidden // 2), torch.uint8)
    scales = Guarded((rows_pad, hidden // 16), torch.uint8)
    if c["resid"]:
        residual = _rows_bf16(g, rows, hidden)
        gate = _vec(g, hidden, 1.0, 0.5)
        bias = _vec(g, hidden, 0.0, 0.05) if c["with_bias"] else None
        r = Guarded((rows, hidden), torch.bfloat16)
        qe.dit_scale_residual_norm_modulate_fp4(
            r.t, y.t, packed.t, scales.t, layout, dev(x), dev(bias), dev(gate), dev(residual),
            dev(scale), dev(shift), dscalar(gv), rows, hidden, c["eps"])
        rr, ry, rp, rs, s_pre, pre = oracle_mod.scale_residual_norm_modulate_fp4(
            bits(x), None if bias is None else bits(bias), bits(gate), bits(residual),
            bits(scale), bits(shift), gv, c["eps"])
        torch.cuda.synchronize()
        r.check("r")
        check_bf16("residual_out", r.bits(), rr)
    else:
        qe.dit_norm_modulate_fp4(y.t, packed.t, scales.t, layout, dev(x), dev(scale),
                                 dev(shift), dscalar(gv), rows, hidden, c["eps"])
        ry, rp, rs, s_pre, pre = oracle_mod.norm_modulate_fp4(bits(x), bits(scale), bits(shift),
                                                              gv, c["eps"])
        torch.cuda.synchronize()
    y.check("y"), packed.check("packed"), scales.check("scales")
    check_bf16("y", y.bits(), ry)
    gs = scales.bits()
    if tiled:
        check_exact("128x4 scales", gs.reshape(-1), oracle_mod.fp4_scales_to_128x4(rs))
        gs = rs
    check_fp4("norm fp4", packed.bits(), gs, rp, rs, s_pre, pre, oracle_mod.f32_from_bf16(ry),
              gv, e4m3_table, oracle_mod.e2m1_encode)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_bias_mul_add(qe, oracle_mod, i):
    rng = np.random.default_rng(4000 + i)
    hidden = 8 * int(rng.integers(1, 3201))
    rows = int(rng.integers(1, max(2, min(2000, 4_000_000 // hidden))))
    with_bias = bool(rng.integers(0, 2))
    _print_case("random bias_mul_add", rows, hidden, with_bias, i)
    g = torch.Generator().manual_seed(5000 + i)
    x, residual = _rows_bf16(g, rows, hidden), _rows_bf16(g, rows, hidden)
    gate = _vec(g, hidden, 0.0, float(10.0 ** rng.uniform(-2, 1)))
    bias = _vec(g, hidden, 0.0, 0.05) if with_bias else None
    y = Guarded((rows, hidden), torch.bfloat16)
    qe.dit_bias_mul_add(y.t, dev(x), dev(bias), dev(gate), dev(residual), rows, hidden)
    ref = oracle_mod.bias_mul_add(bits(x), None if bias is None else bits(bias), bits(gate),
                                  bits(residual))
    torch.cuda.synchronize()
    y.check("y")
    check_bf16("bias_mul_add", y.bits(), ref)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_token_cat(qe, oracle_mod, e4m3_table, i):
    rng = np.random.default_rng(6000 + i)
    a_cols = 16 * int(rng.integers(1, 513))
    b_cols = 16 * int(rng.integers(0, 1537))
    rows = int(rng.integers(1, max(2, min(700, 6_000_000 // (a_cols + b_cols)))))
    fp8_scale = _log_uniform(rng, 1e-3, 1e2)
    g_inv = _log_uniform(rng, 1e-2, 1e4)
    _print_case("random token_cat", rows, a_cols, b_cols, fp8_scale, g_inv, i)
    g = torch.Generator().manual_seed(7000 + i)
    a, b = _rows_bf16(g, rows, a_cols), _rows_bf16(g, rows, b_cols)
    cols = a_cols + b_cols
    out8 = Guarded((rows, cols), torch.uint8)
    qe.dit_token_cat_quant(qe.DIT_QUANT_FP8_E4M3, out8.t, None, dev(a), a_cols, dev(b), b_cols,
                           rows, dscalar(fp8_scale))
    rq, pre = oracle_mod.token_cat_fp8(bits(a), bits(b), fp8_scale)
    rows_pad = (rows + 127) // 128 * 128
    kinds = [(qe.DIT_QUANT_FP4_E2M1, False)]
    if cols % 64 == 0:
        kinds.append((qe.DIT_QUANT_FP4_E2M1_128X4, True))
    rp, rs, s_pre, pre4 = oracle_mod.token_cat_fp4(bits(a), bits(b), g_inv)
    xf = oracle_mod.f32_from_bf16(np.concatenate([bits(a), bits(b)], axis=1))
    torch.cuda.synchronize()
    out8.check("fp8")
    check_fp8("token_cat fp8", out8.bits(), rq, pre, e4m3_table)
    for kind, tiled in kinds:
        packed = Guarded((rows, cols // 2), torch.uint8)
        scales = Guarded((rows_pad, cols // 16), torch.uint8)
        qe.dit_token_cat_quant(kind, packed.t, scales.t, dev(a), a_cols, dev(b), b_cols, rows,
                               dscalar(g_inv))
        torch.cuda.synchronize()
        packed.check("packed"), scales.check("scales")
        gs = scales.bits()
        if tiled:
            check_exact("128x4 scales", gs.reshape(-1), oracle_mod.fp4_scales_to_128x4(rs))
            gs = rs
        check_fp4("token_cat fp4", packed.bits(), gs, rp, rs, s_pre, pre4, xf, g_inv, e4m3_table,
                  oracle_mod.e2m1_encode)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_qkv(qe, oracle_mod, i):
    rng = np.random.default_rng(8000 + i)
    heads = int(rng.integers(1, 65))
    txt_rows, img_rows = int(rng.integers(0, 200)), int(rng.integers(0, 400))
    if txt_rows + img_rows == 0:
        img_rows = 1
    shared = bool(rng.integers(0, 2))
    _print_case("random qkv", img_rows, txt_rows, heads, shared, i)
    g = torch.Generator().manual_seed(9000 + i)
    w = heads * 128
    img = _rows_bf16(g, img_rows, 3 * w)
    txt = _rows_bf16(g, txt_rows, 3 * w)
    ws = [_vec(g, 128, 1.0, float(10.0 ** rng.uniform(-2, 0))) for _ in range(4)]
    # cos/sin: random positions and base, as a cache from any caller would hold
    theta = float(10.0 ** rng.uniform(2, 5))
    pos = rng.integers(0, 100000, size=txt_rows + img_rows)
    tc, ts = synth.rope_tables(pos[:txt_rows], 128, theta)
    ic, is_ = synth.rope_tables(pos[txt_rows:], 128, theta)
    inp = synth.QkvInputs(img, txt, ws[0], ws[1], ws[2], ws[3], ic, is_, tc, ts, heads, 128,
                          float(rng.choice([1e-6, 1e-5, 1e-3])),
                          float(rng.choice([1e-6, 1e-5, 1e-3])))
    gq, gk, gv = _run_qkv(qe, inp, shared_cache=shared)
    rq, rk, rv = _oracle_qkv(oracle_mod, inp)
    check_bf16("joint_q", gq, rq)
    check_bf16("joint_k", gk, rk)
    check_exact("joint_v", gv, rv)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_norm_dual(qe, oracle_mod, e4m3_table, i):
    rng = np.random.default_rng(10000 + i)
    hidden = 8 * int(rng.integers(1, 1025))
    cap = max(2, min(3000, 3_000_000 // hidden))
    img_rows, txt_rows = int(rng.integers(0, cap)), int(rng.integers(0, cap // 4 + 1))
    outs = {"img": str(rng.choice(["yq", "y", "q"])), "txt": str(rng.choice(["yq", "y", "q"]))}
    _print_case("random norm dual", img_rows, txt_rows, hidden, outs, i)
    g = torch.Generator().manual_seed(11000 + i)
    sets = {}
    for name, rows in (("img", img_rows), ("txt", txt_rows)):
        x = _rows_bf16(g, rows, hidden)
        scale, shift = _vec(g, hidden, 0.0, 0.3), _vec(g, hidden, 0.0, 0.3)
        s = _log_uniform(rng, 1e-3, 1e2)
        eps = float(rng.choice([1e-6, 1e-5, 1e-3]))
        y = Guarded((rows, hidden), torch.bfloat16) if "y" in outs[name] else None
        q = Guarded((rows, hidden), torch.uint8) if "q" in outs[name] else None
        sets[name] = (x, scale, shift, s, eps, y, q)
    ptr = lambda o: None if o is None else o.t  # noqa: E731
    (ix, isc, ish, is_, ie, iy, iq), (tx, tsc, tsh, ts, te, ty, tq) = sets["img"], sets["txt"]
    qe.dit_norm_modulate_fp8_dual(ptr(iy), ptr(iq), dev(ix), dev(isc), dev(ish), dscalar(is_),
                                  img_rows, ie, ptr(ty), ptr(tq), dev(tx), dev(tsc), dev(tsh),
                                  dscalar(ts), txt_rows, te, hidden)
    torch.cuda.synchronize()
    for name, (x, scale, shift, s, eps, y, q) in sets.items():
        ry, rq, pre = oracle_mod.norm_modulate_fp8(bits(x), bits(scale), bits(shift), s, eps)
        if y is not None:
            y.check(name + " y")
            check_bf16(name + " y", y.bits(), ry)
        if q is not None:
            q.check(name + " q")
            check_fp8(name + " q", q.bits(), rq, pre, e4m3_table)

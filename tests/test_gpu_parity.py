"""GPU parity: every entry point of libdit_epilogues against the CPU oracle.

Inputs come from `synth` (seeded), the same bytes go to the oracle and to the
GPU, and the outputs are compared with the tolerance rules in parity.py.
Sizes cover the full workload shapes (512 text + 4096 image tokens, hidden
3072, 24 heads; FLUX.2 rows of 6144 + 18432) and small ragged cases: partial
waves and workgroups, hidden sizes that are not multiples of 512, heads not
multiples of 4 and above 24, pad rows of the FP4 scale matrix. Outputs sit
between guard bytes that must survive every call.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import parity
import synth
from parity import check_exact

pytestmark = pytest.mark.gpu


# Every case below is bit-exact against the oracle. Each check first applies
# the tolerance rule (parity.py), then requires every output byte to be
# equal, so a failure says which of the two bars was missed.
def check_bf16(name, gpu, ref):
    return parity.check_bf16(name, gpu, ref, exact=True)


def check_fp8(name, gpu, ref, pre, table):
    return parity.check_fp8(name, gpu, ref, pre, table, exact=True)


def check_fp4(*args):
    return parity.check_fp4(*args, exact=True)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _row_slices(rows: int, n: int):
    return [(rows * k // n, rows * (k + 1) // n) for k in range(n) if rows * k // n < rows * (k + 1) // n]


def _parallel(fn, rows: int):
    """fn(lo, hi) over contiguous row slices on a thread pool (the oracle's C
    entry points release Python's lock); returns the results in row order."""
    with ThreadPoolExecutor(_threads()) as ex:
        return list(ex.map(lambda lh: fn(*lh), _row_slices(rows, 4 * _threads())))

GUARD = 4096  # bytes on each side of every output buffer


@pytest.fixture(scope="module")
def qe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import quant_epilogues_amd as qe_mod

    qe_mod.lib()  # raises if the HIP library is not built
    return qe_mod


@pytest.fixture(scope="module")
def e4m3_table(oracle_mod):
    return oracle_mod.e4m3_decode(np.arange(256, dtype=np.uint8))


class Guarded:
    """A device output tensor framed by canary bytes."""

    def __init__(self, shape, dtype):
        n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        self.n = n
        self.buf = torch.full((n + 2 * GUARD,), 0xA5, dtype=torch.uint8, device="cuda")
        self.t = self.buf[GUARD:GUARD + n].view(dtype).view(shape)

    def check(self, name):
        head = self.buf[:GUARD].cpu().numpy()
        tail = self.buf[GUARD + self.n:].cpu().numpy()
        assert np.all(head == 0xA5) and np.all(tail == 0xA5), f"{name}: write outside its buffer"

    def bits(self):
        t = self.t.cpu()
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).numpy().view(np.uint16)
        return t.numpy()


def dev(t):
    return t.cuda() if t is not None else None


def dscalar(v):
    return torch.tensor([v], dtype=torch.float32, device="cuda")


def bits(t):
    return synth.bf16_bits(t)


def _print_case(*args):
    print("case:", *args, flush=True)


# ---------------------------------------------------------------------------
# LayerNorm + modulation + FP8
# ---------------------------------------------------------------------------

NORM_CASES = [
    (127, 3072, 0.0625, 0),   # the small Qwen-Image case
    (512, 3072, 0.0625, 11),  # Qwen-Image text tokens, as bench.py launches them
    (1, 3072, 0.4754464328, 1),
    (1024, 3072, 0.02, 2),
    (4096, 3072, 0.5, 3),     # full image-token count
    (33, 512, 0.0625, 4),
    (17, 1000, 0.0625, 5),    # ragged: 125 chunks, a partial last wave
    (9, 6144, 0.02, 6),       # FLUX.2 width, 12 waves per row
    (1024, 6144, 0.0625, 9),  # FLUX.2 width, many rows: six waves per row
    (1030, 4104, 0.5, 10),    # 513 chunks per row: a partial last wave
    (3, 8192, 0.0625, 8),     # widest supported row: 1024 threads
    (5, 8, 0.0625, 7),        # one chunk per row
    (4608, 3072, 0.0625, 12),  # 4097..6144 rows: one wave per row, one resident round
    (6144, 2736, 0.02, 13),    # the same geometry at its row limit, 342 chunks (ragged)
]


@pytest.mark.parametrize("rows,hidden,input_scale,seed", NORM_CASES)
def test_norm_modulate_fp8(qe, oracle_mod, e4m3_table, rows, hidden, input_scale, seed):
    _print_case("norm_modulate_fp8", rows, hidden, input_scale, seed)
    inp = synth.norm_modulate_inputs(rows, hidden, seed=seed, input_scale=input_scale)
    y = Guarded((rows, hidden), torch.bfloat16)
    q = Guarded((rows, hidden), torch.uint8)
    qe.dit_norm_modulate_fp8(y.t, q.t, dev(inp.x), dev(inp.scale), dev(inp.shift),
                             dscalar(inp.input_scale), rows, hidden, inp.eps)
    torch.cuda.synchronize()
    y.check("y"), q.check("q")
    ry, rq, pre = oracle_mod.norm_modulate_fp8(bits(inp.x), bits(inp.scale), bits(inp.shift),
                                               inp.input_scale, inp.eps)
    ey = check_bf16("y", y.bits(), ry)
    eq = check_fp8("q", q.bits(), rq, pre, e4m3_table)
    print(f"exact: y {ey:.6f} q {eq:.6f}")


DUAL_CASES = [
    # (img_rows, txt_rows, hidden, img_scale, txt_scale, img_eps, txt_eps, seed)
    (4096, 512, 3072, 0.0625, 0.02, 1e-6, 1e-5, 60),  # Qwen-Image: 4096 image + 512 text tokens
    (1000, 30, 3072, 0.5, 0.0625, 1e-6, 0.25, 61),    # partial last workgroup in both sets
    (600, 300, 3072, 0.02, 0.5, 1e-6, 1e-6, 62),      # under 1024 rows in all: the latency geometry
    (9, 1030, 6144, 0.0625, 0.02, 1e-5, 1e-6, 63),    # FLUX.2 width
    (33, 17, 1000, 0.0625, 0.5, 1e-6, 1e-6, 64),      # ragged width: 125 chunks
    (4000, 1000, 2736, 0.5, 0.02, 1e-6, 1e-5, 69),    # one wave per row, ragged width
    (0, 77, 3072, 0.0625, 0.02, 1e-6, 1e-6, 65),      # no image rows
    (1030, 0, 3072, 0.0625, 0.02, 1e-6, 1e-6, 66),    # no text rows
]


@pytest.mark.parametrize("img_rows,txt_rows,hidden,img_s,txt_s,img_eps,txt_eps,seed", DUAL_CASES)
def test_norm_modulate_fp8_dual(qe, oracle_mod, e4m3_table, img_rows, txt_rows, hidden, img_s,
                                txt_s, img_eps, txt_eps, seed):
    """Image and text rows in one launch, each with its own vectors, FP8 scale
    and eps: each stream equals the oracle on that stream alone."""
    _print_case("norm_modulate_fp8_dual", img_rows, txt_rows, hidden, seed)
    img = synth.norm_modulate_inputs(img_rows, hidden, seed=seed, input_scale=img_s, eps=img_eps)
    txt = synth.norm_modulate_inputs(txt_rows, hidden, seed=seed + 1000, input_scale=txt_s,
                                     eps=txt_eps)
    out = {}
    for name, rows in (("img", img_rows), ("txt", txt_rows)):
        out[name] = (Guarded((rows, hidden), torch.bfloat16), Guarded((rows, hidden), torch.uint8))
    (iy, iq), (ty, tq) = out["img"], out["txt"]
    qe.dit_norm_modulate_fp8_dual(
        iy.t, iq.t, dev(img.x), dev(img.scale), dev(img.shift), dscalar(img.input_scale), img_rows,
        img.eps, ty.t, tq.t, dev(txt.x), dev(txt.scale), dev(txt.shift), dscalar(txt.input_scale),
        txt_rows, txt.eps, hidden)
    torch.cuda.synchronize()
    for name, inp in (("img", img), ("txt", txt)):
        y, q = out[name]
        y.check(name + " y"), q.check(name + " q")
        ry, rq, pre = oracle_mod.norm_modulate_fp8(bits(inp.x), bits(inp.scale), bits(inp.shift),
                                                   inp.input_scale, inp.eps)
        check_bf16(name + " y", y.bits(), ry)
        check_fp8(name + " q", q.bits(), rq, pre, e4m3_table)
    print("exact: y 1.000000 q 1.000000 (both streams)")


def test_norm_modulate_fp8_dual_equals_two_calls(qe):
    """The one-launch form and two single-stream calls give the same bytes,
    including with one output left out."""
    img = synth.norm_modulate_inputs(512, 3072, seed=67, input_scale=0.02)
    txt = synth.norm_modulate_inputs(128, 3072, seed=68, input_scale=0.5, eps=1e-5)
    args = lambda i: (dev(i.x), dev(i.scale), dev(i.shift), dscalar(i.input_scale))
    for want_y, want_q in ((True, True), (False, True), (True, False)):
        (yi, qi), (yt, qt) = qe.norm_modulate_fp8_dual(*args(img), *args(txt), img.eps, txt.eps,
                                                       want_y=want_y, want_q=want_q)
        yi2, qi2 = qe.norm_modulate_fp8(*args(img), img.eps, want_y=want_y, want_q=want_q)
        yt2, qt2 = qe.norm_modulate_fp8(*args(txt), txt.eps, want_y=want_y, want_q=want_q)
        torch.cuda.synchronize()
        for a, b in ((yi, yi2), (qi, qi2), (yt, yt2), (qt, qt2)):
            assert (a is None) == (b is None)
            if a is not None:
                assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))


DUAL_SELECT_CASES = [
    # (img_rows, txt_rows, hidden, img outputs, txt outputs, seed); the geometry
    # at 6144 follows whether the text rows (the first set) write y
    (1000, 200, 3072, "yq", "q", 70),
    (1000, 200, 3072, "q", "y", 71),
    (2000, 100, 6144, "y", "q", 72),
    (2000, 100, 6144, "q", "yq", 73),
]


@pytest.mark.parametrize("img_rows,txt_rows,hidden,img_out,txt_out,seed", DUAL_SELECT_CASES)
def test_norm_modulate_fp8_dual_output_selection(qe, oracle_mod, e4m3_table, img_rows, txt_rows,
                                                 hidden, img_out, txt_out, seed):
    """Each row set of the one-launch norm writes only the outputs it asks for,
    and those equal the oracle's."""
    _print_case("norm_modulate_fp8_dual selection", img_rows, txt_rows, hidden, img_out, txt_out,
                seed)
    img = synth.norm_modulate_inputs(img_rows, hidden, seed=seed, input_scale=0.0625)
    txt = synth.norm_modulate_inputs(txt_rows, hidden, seed=seed + 1000, input_scale=0.02,
                                     eps=1e-5)
    out = {}
    for name, rows, sel in (("img", img_rows, img_out), ("txt", txt_rows, txt_out)):
        out[name] = (Guarded((rows, hidden), torch.bfloat16) if "y" in sel else None,
                     Guarded((rows, hidden), torch.uint8) if "q" in sel else None)
    ptr = lambda g: None if g is None else g.t
    (iy, iq), (ty, tq) = out["img"], out["txt"]
    qe.dit_norm_modulate_fp8_dual(
        ptr(iy), ptr(iq), dev(img.x), dev(img.scale), dev(img.shift), dscalar(img.input_scale),
        img_rows, img.eps, ptr(ty), ptr(tq), dev(txt.x), dev(txt.scale), dev(txt.shift),
        dscalar(txt.input_scale), txt_rows, txt.eps, hidden)
    torch.cuda.synchronize()
    for name, inp in (("img", img), ("txt", txt)):
        y, q = out[name]
        ry, rq, pre = oracle_mod.norm_modulate_fp8(bits(inp.x), bits(inp.scale), bits(inp.shift),
                                                   inp.input_scale, inp.eps)
        if y is not None:
            y.check(name + " y")
            check_bf16(name + " y", y.bits(), ry)
        if q is not None:
            q.check(name + " q")
            check_fp8(name + " q", q.bits(), rq, pre, e4m3_table)


SR_CASES = [
    (4096, 3072, 0.02, True, 0),
    (4096, 3072, 0.0625, True, 1),
    (4096, 3072, 0.5, True, 2),
    (4096, 3072, 0.0625, False, 3),
    (127, 3072, 0.0625, True, 4),
    (13, 1000, 0.02, True, 5),
    (6, 6144, 0.5, False, 6),
]


@pytest.mark.parametrize("rows,hidden,input_scale,with_bias,seed", SR_CASES)
def test_scale_residual_norm_modulate_fp8(qe, oracle_mod, e4m3_table, rows, hidden,
                                          input_scale, with_bias, seed):
    _print_case("scale_residual", rows, hidden, input_scale, with_bias, seed)
    inp = synth.scale_residual_inputs(rows, hidden, seed=seed, input_scale=input_scale,
                                      with_bias=with_bias)
    r = Guarded((rows, hidden), torch.bfloat16)
    y = Guarded((rows, hidden), torch.bfloat16)
    q = Guarded((rows, hidden), torch.uint8)
    qe.dit_scale_residual_norm_modulate_fp8(
        r.t, y.t, q.t, dev(inp.x), dev(inp.bias), dev(inp.gate), dev(inp.residual),
        dev(inp.scale), dev(inp.shift), dscalar(inp.input_scale), rows, hidden, inp.eps)
    torch.cuda.synchronize()
    for o, n in ((r, "r"), (y, "y"), (q, "q")):
        o.check(n)
    rr, ry, rq, pre = oracle_mod.scale_residual_norm_modulate_fp8(
        bits(inp.x), None if inp.bias is None else bits(inp.bias), bits(inp.gate),
        bits(inp.residual), bits(inp.scale), bits(inp.shift), inp.input_scale, inp.eps)
    er = check_bf16("residual_out", r.bits(), rr)
    ey = check_bf16("y", y.bits(), ry)
    eq = check_fp8("q", q.bits(), rq, pre, e4m3_table)
    print(f"exact: r {er:.6f} y {ey:.6f} q {eq:.6f}")


SELECT_CASES = [
    # (rows, hidden, input_scale, residual variant, with_bias, write y, write q, seed)
    (4608, 6144, 0.0625, False, False, False, True, 30),  # FLUX.2 LN + modulate, FP8 only
    (4096, 3072, 0.0625, True, True, True, False, 31),    # Qwen-Image bias + residual norm, bf16 only
    (4096, 3072, 0.02, True, True, False, True, 32),
    (127, 3072, 0.0625, False, False, True, False, 33),
    (17, 1000, 0.5, True, False, False, True, 34),
    (1030, 4104, 0.0625, False, False, False, True, 35),  # FP8 only, 513 chunks per row
    (1031, 6144, 0.5, False, False, False, True, 36),     # scale/shift parked in LDS; the last
                                                          # workgroup's second row slot is empty
]


@pytest.mark.parametrize("rows,hidden,input_scale,resid,with_bias,want_y,want_q,seed", SELECT_CASES)
def test_norm_output_selection(qe, oracle_mod, e4m3_table, rows, hidden, input_scale, resid,
                               with_bias, want_y, want_q, seed):
    """One of the two outputs not requested (NULL): the other is unchanged."""
    _print_case("norm output selection", rows, hidden, input_scale, resid, with_bias, want_y,
                want_q, seed)
    y = Guarded((rows, hidden), torch.bfloat16) if want_y else None
    q = Guarded((rows, hidden), torch.uint8) if want_q else None
    s = dscalar(input_scale) if want_q else None
    if resid:
        inp = synth.scale_residual_inputs(rows, hidden, seed=seed, input_scale=input_scale,
                                          with_bias=with_bias)
        r = Guarded((rows, hidden), torch.bfloat16)
        qe.dit_scale_residual_norm_modulate_fp8(
            r.t, y and y.t, q and q.t, dev(inp.x), dev(inp.bias), dev(inp.gate),
            dev(inp.residual), dev(inp.scale), dev(inp.shift), s, rows, hidden, inp.eps)
        rr, ry, rq, pre = oracle_mod.scale_residual_norm_modulate_fp8(
            bits(inp.x), None if inp.bias is None else bits(inp.bias), bits(inp.gate),
            bits(inp.residual), bits(inp.scale), bits(inp.shift), inp.input_scale, inp.eps)
    else:
        inp = synth.norm_modulate_inputs(rows, hidden, seed=seed, input_scale=input_scale)
        qe.dit_norm_modulate_fp8(y and y.t, q and q.t, dev(inp.x), dev(inp.scale),
                                 dev(inp.shift), s, rows, hidden, inp.eps)
        ry, rq, pre = oracle_mod.norm_modulate_fp8(bits(inp.x), bits(inp.scale),
                                                   bits(inp.shift), inp.input_scale, inp.eps)
    torch.cuda.synchronize()
    msg = []
    if resid:
        r.check("r")
        msg.append(f"r {check_bf16('residual_out', r.bits(), rr):.6f}")
    if want_y:
        y.check("y")
        msg.append(f"y {check_bf16('y', y.bits(), ry):.6f}")
    if want_q:
        q.check("q")
        msg.append(f"q {check_fp8('q', q.bits(), rq, pre, e4m3_table):.6f}")
    print("exact: " + " ".join(msg))


NORM_FP4_CASES = [
    # (rows, hidden, residual variant, with_bias, write y, g, 128x4 scales, seed)
    (4096, 3072, True, True, True, 448.0, False, 40),    # Qwen-Image bias + residual norm
    (4096, 3072, True, True, False, 448.0, True, 47),    # the same, 128x4 scales, FP4 only
    (4608, 6144, False, False, False, 448.0, False, 41),  # FLUX.2 width, FP4 only
    (127, 3072, False, False, True, 1.0, True, 42),       # one partial 128-row tile
    (17, 1008, True, False, True, 448.0, False, 43),     # 111 pad rows, 126 chunks: a ragged wave
    (5, 16, False, False, True, 1e4, False, 44),         # one group per row, saturating scales
    (1030, 4112, False, False, True, 448.0, False, 45),  # 514 chunks per row, six-wave geometry
    (1030, 4112, True, True, False, 448.0, False, 46),
    (300, 4096, False, False, True, 448.0, True, 48),    # three row tiles, 64 tile columns
]


@pytest.mark.parametrize("rows,hidden,resid,with_bias,want_y,g,tiled,seed", NORM_FP4_CASES)
def test_norm_fp4(qe, oracle_mod, e4m3_table, rows, hidden, resid, with_bias, want_y, g, tiled,
                  seed):
    """LayerNorm (optionally after bias + gated residual) with NVFP4 output; the
    128x4 scale layout is checked as the oracle's row-major scales rearranged."""
    _print_case("norm fp4", rows, hidden, resid, with_bias, want_y, g, tiled, seed)
    layout = qe.DIT_FP4_SCALES_128X4 if tiled else qe.DIT_FP4_SCALES_ROW_MAJOR
    gv = float(np.float32(g))
    rows_pad = (rows + 127) // 128 * 128
    y = Guarded((rows, hidden), torch.bfloat16) if want_y else None
    packed = Guarded((rows, hidden // 2), torch.uint8)
    scales = Guarded((rows_pad, hidden // 16), torch.uint8)
    if resid:
        inp = synth.scale_residual_inputs(rows, hidden, seed=seed, with_bias=with_bias)
        r = Guarded((rows, hidden), torch.bfloat16)
        qe.dit_scale_residual_norm_modulate_fp4(
            r.t, y and y.t, packed.t, scales.t, layout, dev(inp.x), dev(inp.bias), dev(inp.gate),
            dev(inp.residual), dev(inp.scale), dev(inp.shift), dscalar(gv), rows, hidden, inp.eps)
        rr, ry, rp, rs, s_pre, pre = oracle_mod.scale_residual_norm_modulate_fp4(
            bits(inp.x), None if inp.bias is None else bits(inp.bias), bits(inp.gate),
            bits(inp.residual), bits(inp.scale), bits(inp.shift), gv, inp.eps)
    else:
        inp = synth.norm_modulate_inputs(rows, hidden, seed=seed)
        qe.dit_norm_modulate_fp4(y and y.t, packed.t, scales.t, layout, dev(inp.x),
                                 dev(inp.scale), dev(inp.shift), dscalar(gv), rows, hidden, inp.eps)
        ry, rp, rs, s_pre, pre = oracle_mod.norm_modulate_fp4(
            bits(inp.x), bits(inp.scale), bits(inp.shift), gv, inp.eps)
    torch.cuda.synchronize()
    msg = []
    if resid:
        r.check("r")
        msg.append(f"r {check_bf16('residual_out', r.bits(), rr):.6f}")
    if want_y:
        y.check("y")
        msg.append(f"y {check_bf16('y', y.bits(), ry):.6f}")
    packed.check("packed"), scales.check("scales")
    gs = scales.bits()
    if tiled:  # the same scale bytes, rearranged: compare in the tile layout
        check_exact("128x4 scales", gs.reshape(-1), oracle_mod.fp4_scales_to_128x4(rs))
        gs = rs  # the codes are then checked against the row-major scales
    ec, es = check_fp4("norm fp4", packed.bits(), gs, rp, rs, s_pre, pre,
                       oracle_mod.f32_from_bf16(ry), gv, e4m3_table, oracle_mod.e2m1_encode)
    msg.append(f"codes {ec:.6f} scales {es:.6f}")
    print("exact: " + " ".join(msg))


# Widths whose chunks per row (66, 130, 260, 384, 450, 700, 800) land in every
# case of the norm launcher's width switches: one, two and three chunks per
# lane at two waves per row (384: the exact fit), the six-wave plain geometry,
# eight chunks per lane, one-wave residual rows with 2..6 chunks per lane and
# the two-wave residual geometry with 4, 6 and 8; at 37 rows the latency path
# with one, two and three chunks per lane.
GEOMETRY_WIDTHS = [528, 1040, 2080, 3072, 3600, 5600, 6400]


@pytest.mark.parametrize("rows", [1031, 37])
@pytest.mark.parametrize("hidden", GEOMETRY_WIDTHS)
def test_norm_every_geometry(qe, oracle_mod, e4m3_table, rows, hidden):
    """Every kernel instance the norm launcher can pick for these widths, at a
    row count on the many-rows path (1031: a partial last workgroup) and one
    on the latency path (37): the plain norm and both residual variants with
    both outputs, and NVFP4 output with and without the residual (128x4
    scales where the width allows)."""
    seed = 7 * hidden + rows
    test_norm_output_selection(qe, oracle_mod, e4m3_table, rows, hidden, 0.0625,
                               False, False, True, True, seed)
    test_norm_output_selection(qe, oracle_mod, e4m3_table, rows, hidden, 0.0625,
                               True, True, True, True, seed + 1)
    test_norm_output_selection(qe, oracle_mod, e4m3_table, rows, hidden, 0.0625,
                               True, False, True, True, seed + 2)
    test_norm_fp4(qe, oracle_mod, e4m3_table, rows, hidden, True, True, True, 448.0, False,
                  seed + 3)
    test_norm_fp4(qe, oracle_mod, e4m3_table, rows, hidden, False, False, True, 448.0,
                  hidden % 64 == 0, seed + 4)


def test_fp8_split_equals_fused_on_gpu(qe):
    """q of the fused kernel == y re-quantised by the token-cat FP8 path."""
    inp = synth.norm_modulate_inputs(256, 3072, seed=21, input_scale=0.4754464328)
    s = dscalar(inp.input_scale)
    y, q = qe.norm_modulate_fp8(dev(inp.x), dev(inp.scale), dev(inp.shift), s, inp.eps)
    q2 = qe.token_cat_quant(qe.DIT_QUANT_FP8_E4M3, y, None, s)
    torch.cuda.synchronize()
    assert torch.equal(q.cpu(), q2.cpu())


# ---------------------------------------------------------------------------
# QKV epilogue
# ---------------------------------------------------------------------------

QKV_CASES = [
    (4096, 512, 24, 0, False),   # Qwen-Image 1024^2: 4096 image + 512 text tokens
    (5, 3, 3, 1, False),         # heads not a multiple of 4
    (7, 2, 24, 2, False),
    (3, 4, 48, 3, True),         # FLUX.2 head count (four 12-head waves), shared cache
    (2, 1, 64, 4, False),
    (6, 0, 24, 5, True),         # image only
    (0, 5, 5, 6, True),          # text only
    (3, 2, 30, 7, False),        # three head groups, the last one partial
    (2, 3, 60, 8, True),         # five head groups
]


def _run_qkv(qe, inp, contiguous=False, shared_cache=False):
    """Runs the C entry point. shared_cache: the four cos/sin tables are views
    of one [txt + img, 128] fp32 cache whose rows hold [cos | sin] in joint
    order (row stride 128), as the FLUX.2 variant binds them."""
    views = {}
    for stream in ("img", "txt"):
        qkv = dev(inp.img_qkv if stream == "img" else inp.txt_qkv)
        q, k, v = inp.width, 2 * inp.width, 3 * inp.width
        vs = (qkv[:, 0:q], qkv[:, q:k], qkv[:, k:v])
        if contiguous:
            vs = tuple(t.contiguous() for t in vs)
        views[stream] = vs
    n_txt, n = inp.txt_qkv.shape[0], inp.img_qkv.shape[0] + inp.txt_qkv.shape[0]
    outs = [Guarded((n, inp.heads, inp.head_dim), torch.bfloat16) for _ in range(3)]
    half = inp.head_dim // 2
    if shared_cache:
        cache = np.concatenate([np.concatenate([inp.txt_cos, inp.txt_sin], axis=1),
                                np.concatenate([inp.img_cos, inp.img_sin], axis=1)])
        cache = torch.from_numpy(np.ascontiguousarray(cache, np.float32)).cuda()
        tables = (cache[n_txt:, :half], cache[n_txt:, half:], cache[:n_txt, :half],
                  cache[:n_txt, half:])
        stride = 2 * half
    else:
        tables = tuple(torch.from_numpy(np.ascontiguousarray(t)).cuda()
                       for t in (inp.img_cos, inp.img_sin, inp.txt_cos, inp.txt_sin))
        stride = half
    (iq, ik, iv), (tq, tk, tv) = views["img"], views["txt"]
    qe.dit_qkv_epilogue(outs[0].t, outs[1].t, outs[2].t, iq, ik, iv, iq.shape[0], iq.stride(0),
                        tq, tk, tv, tq.shape[0], tq.stride(0), dev(inp.img_q_w),
                        dev(inp.img_k_w), dev(inp.txt_q_w), dev(inp.txt_k_w), *tables, stride,
                        inp.heads, inp.head_dim, inp.img_eps, inp.txt_eps)
    torch.cuda.synchronize()
    for o, name in zip(outs, "qkv"):
        o.check("joint_" + name)
    return [o.bits() for o in outs]


def _oracle_qkv(oracle_mod, inp, img_sel=None, txt_sel=None):
    """The oracle on all rows, or on the selected image / text rows (joint
    output rows: the selected text rows, then the selected image rows)."""
    i_sel = np.arange(inp.img_qkv.shape[0]) if img_sel is None else img_sel
    t_sel = np.arange(inp.txt_qkv.shape[0]) if txt_sel is None else txt_sel
    return oracle_mod.qkv_epilogue_packed(
        bits(inp.img_qkv)[i_sel], bits(inp.txt_qkv)[t_sel], bits(inp.img_q_w),
        bits(inp.img_k_w), bits(inp.txt_q_w), bits(inp.txt_k_w), inp.img_cos[i_sel],
        inp.img_sin[i_sel], inp.txt_cos[t_sel], inp.txt_sin[t_sel], inp.heads, inp.head_dim,
        inp.img_eps, inp.txt_eps)


@pytest.mark.parametrize("img_rows,txt_rows,heads,seed,shared", QKV_CASES)
def test_qkv_epilogue(qe, oracle_mod, img_rows, txt_rows, heads, seed, shared):
    _print_case("qkv_epilogue", img_rows, txt_rows, heads, seed, shared)
    inp = synth.qkv_inputs(img_rows, txt_rows, heads, 128, seed=seed, img_eps=1e-6,
                           txt_eps=1e-5)
    gq, gk, gv = _run_qkv(qe, inp, shared_cache=shared)
    rq, rk, rv = _oracle_qkv(oracle_mod, inp)
    eq = check_bf16("joint_q", gq, rq)
    ek = check_bf16("joint_k", gk, rk)
    check_exact("joint_v", gv, rv)
    print(f"exact: q {eq:.6f} k {ek:.6f}")


def test_qkv_epilogue_flux2_full_shape(qe, oracle_mod):
    """FLUX.2 at 1024^2: 4096 image + 512 text tokens, 48 heads, one shared
    [cos | sin] cache; every token of both streams against the oracle (run on
    row slices in parallel)."""
    _print_case("qkv_epilogue flux2", 4096, 512, 48, 11, True)
    inp = synth.qkv_inputs(4096, 512, 48, 128, seed=11, img_eps=1e-6, txt_eps=1e-6)
    gq, gk, gv = _run_qkv(qe, inp, shared_cache=True)
    empty = np.arange(0)

    def img_slice(lo, hi):
        rq, rk, rv = _oracle_qkv(oracle_mod, inp, np.arange(lo, hi), empty)
        sl = slice(512 + lo, 512 + hi)
        check_bf16("joint_q", gq[sl], rq)
        check_bf16("joint_k", gk[sl], rk)
        check_exact("joint_v", gv[sl], rv)

    rq, rk, rv = _oracle_qkv(oracle_mod, inp, empty, np.arange(512))
    check_bf16("joint_q (text)", gq[:512], rq)
    check_bf16("joint_k (text)", gk[:512], rk)
    check_exact("joint_v (text)", gv[:512], rv)
    _parallel(img_slice, 4096)
    print("exact: q 1.000000 k 1.000000 (all 4608 tokens)")


def test_qkv_contiguous_equals_strided(qe):
    inp = synth.qkv_inputs(64, 16, 24, 128, seed=9)
    a = _run_qkv(qe, inp, contiguous=False)
    b = _run_qkv(qe, inp, contiguous=True)
    c = _run_qkv(qe, inp, shared_cache=True)
    for x, y, z in zip(a, b, c):
        assert np.array_equal(x, y) and np.array_equal(x, z)


# ---------------------------------------------------------------------------
# bias_mul_add
# ---------------------------------------------------------------------------

BMA_CASES = [
    (4608, 3072, True, 0),   # 512 text + 4096 image tokens
    (4608, 3072, False, 1),
    (3, 1000, True, 2),
    (5, 6144, True, 3),
    (1, 8, True, 4),
    (2, 25600, True, 5),     # a row longer than one 1024-thread pass
]


@pytest.mark.parametrize("rows,hidden,with_bias,seed", BMA_CASES)
def test_bias_mul_add(qe, oracle_mod, rows, hidden, with_bias, seed):
    _print_case("bias_mul_add", rows, hidden, with_bias, seed)
    inp = synth.bias_mul_add_inputs(rows, hidden, seed=seed, with_bias=with_bias)
    y = Guarded((rows, hidden), torch.bfloat16)
    qe.dit_bias_mul_add(y.t, dev(inp.x), dev(inp.bias), dev(inp.gate), dev(inp.residual),
                        rows, hidden)
    torch.cuda.synchronize()
    y.check("y")
    ry = oracle_mod.bias_mul_add(bits(inp.x), None if inp.bias is None else bits(inp.bias),
                                 bits(inp.gate), bits(inp.residual))
    print(f"exact: y {check_bf16('y', y.bits(), ry):.6f}")


def test_bias_mul_add_tie_case(qe, oracle_mod):
    """The tie-guard inputs of the output-bias-absorption page, on the GPU."""
    import json
    import os

    with open(os.path.join(os.path.dirname(__file__), "golden", "bias_mul_add_tie.json")) as f:
        c = json.load(f)["inputs"]
    H = 8
    t = lambda v: torch.full((1, H), v, dtype=torch.bfloat16)
    x, res = t(c["x"]), t(c["residual"])
    bias, gate = t(c["bias"])[0], t(c["gate"])[0]
    y = qe.bias_mul_add(dev(x), dev(bias), dev(gate), dev(res))
    ry = oracle_mod.bias_mul_add(bits(x), bits(bias), bits(gate), bits(res))
    got = y.cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ry)


# ---------------------------------------------------------------------------
# Token concatenation + FP8 / FP4
# ---------------------------------------------------------------------------

FP8_CASES = [
    (4608, 6144, 18432, 0.05, 0),  # FLUX.2 single block
    (7, 96, 160, 0.05, 1),
    (3, 6144, 0, 0.5, 2),
    (130, 16, 48, 0.4754464328, 3),
    (5, 6144, 2064, 0.05, 7),         # 1026 chunks: three tiles, the last ragged
    (65540, 16, 16, 0.05, 8),         # rows beyond one launch's 65536
]


@pytest.mark.parametrize("rows,a_cols,b_cols,scale,seed", FP8_CASES)
def test_token_cat_fp8(qe, oracle_mod, e4m3_table, rows, a_cols, b_cols, scale, seed):
    """Every row against the oracle (run on row slices in parallel)."""
    _print_case("token_cat_fp8", rows, a_cols, b_cols, scale, seed)
    inp = synth.token_cat_inputs(rows, a_cols, b_cols, seed=seed, fp8_scale=scale)
    cols = a_cols + b_cols
    out = Guarded((rows, cols), torch.uint8)
    qe.dit_token_cat_quant(qe.DIT_QUANT_FP8_E4M3, out.t, None, dev(inp.attn), a_cols,
                           dev(inp.mlp) if b_cols else None, b_cols, rows, dscalar(inp.fp8_scale))
    torch.cuda.synchronize()
    out.check("out")
    got, a_b, m_b = out.bits(), bits(inp.attn), bits(inp.mlp)

    def rows_check(lo, hi):
        rq, pre = oracle_mod.token_cat_fp8(a_b[lo:hi], m_b[lo:hi], inp.fp8_scale)
        return check_fp8(f"q rows {lo}:{hi}", got[lo:hi], rq, pre, e4m3_table)

    _parallel(rows_check, rows)
    print("exact: q 1.000000")


@pytest.mark.parametrize("inv_scale", [1.0, 16.0, 50.0, 20.0, 2.0, 1.0 / 0.4754464328])
def test_token_cat_fp8_all_bf16_values(qe, oracle_mod, inv_scale):
    """Every finite bf16 pattern through the FP8 path, at each scale."""
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    pats = pats[(pats & 0x7F80) != 0x7F80]
    pats = np.concatenate([pats, np.zeros((-pats.size) % 4096, np.uint16)]).reshape(-1, 4096)
    a = torch.from_numpy(pats.view(np.int16)).view(torch.bfloat16)
    scale = float(np.float32(1.0) / np.float32(inv_scale))
    q = qe.token_cat_quant(qe.DIT_QUANT_FP8_E4M3, dev(a), None, dscalar(scale))
    rq, _ = oracle_mod.token_cat_fp8(pats, np.zeros((pats.shape[0], 0), np.uint16), scale)
    check_exact("q", q.cpu().numpy(), rq)


FP4_CASES = [
    (4608, 6144, 18432, "calibrated", 0),
    (17, 64, 192, "calibrated", 1),   # 111 pad rows in the scale matrix
    (9, 32, 32, 1.0, 2),
    (9, 32, 32, 1e4, 3),              # saturating scales
    (128, 6144, 0, "calibrated", 4),
    (129, 16, 16, "calibrated", 5),
    (19, 4112, 4112, "calibrated", 6),  # 514 groups: three tiles, the last ragged
    (65540, 16, 16, "calibrated", 7),   # 65664 scale rows: two launches
]


def _check_fp4_rows(oracle_mod, e4m3_table, name, packed, scales, a_b, m_b, g):
    """Every row's codes and scales (row-major) and the pad-row scales against
    the oracle, on row slices in parallel."""
    rows = packed.shape[0]
    check_exact(name + " pad scales", scales[rows:], np.zeros_like(scales[rows:]))

    def rows_check(lo, hi):
        rp, rs, s_pre, pre = oracle_mod.token_cat_fp4(a_b[lo:hi], m_b[lo:hi], g)
        x = oracle_mod.f32_from_bf16(np.concatenate([a_b[lo:hi], m_b[lo:hi]], axis=1))
        return check_fp4(f"{name} rows {lo}:{hi}", packed[lo:hi], scales[lo:hi], rp,
                         rs[:hi - lo], s_pre, pre, x, g, e4m3_table, oracle_mod.e2m1_encode)

    _parallel(rows_check, rows)


@pytest.mark.parametrize("rows,a_cols,b_cols,g,seed", FP4_CASES)
def test_token_cat_fp4(qe, oracle_mod, e4m3_table, rows, a_cols, b_cols, g, seed):
    _print_case("token_cat_fp4", rows, a_cols, b_cols, g, seed)
    inp = synth.token_cat_inputs(rows, a_cols, b_cols, seed=seed)
    gv = inp.fp4_g if g == "calibrated" else float(np.float32(g))
    cols = a_cols + b_cols
    rows_pad = (rows + 127) // 128 * 128
    packed = Guarded((rows, cols // 2), torch.uint8)
    scales = Guarded((rows_pad, cols // 16), torch.uint8)
    qe.dit_token_cat_quant(qe.DIT_QUANT_FP4_E2M1, packed.t, scales.t, dev(inp.attn), a_cols,
                           dev(inp.mlp) if b_cols else None, b_cols, rows, dscalar(gv))
    torch.cuda.synchronize()
    packed.check("packed"), scales.check("scales")
    _check_fp4_rows(oracle_mod, e4m3_table, "fp4", packed.bits(), scales.bits(),
                    bits(inp.attn), bits(inp.mlp), gv)
    print("exact: codes 1.000000 scales 1.000000")


FP4_128X4_CASES = [
    (4608, 6144, 18432, 50),  # FLUX.2 single block
    (130, 64, 192, 51),       # 16 groups: one workgroup's four tile columns; two row tiles
    (33, 64, 128, 52),        # 12 groups: a workgroup with three of its four tile columns
    (300, 1024, 1088, 53),    # 132 groups: the last workgroup holds one tile column; three row tiles
    (129, 6144, 64, 54),      # 388 groups, the branch boundary inside a wave's span
]


@pytest.mark.parametrize("rows,a_cols,b_cols,seed", FP4_128X4_CASES)
def test_token_cat_fp4_128x4_scales(qe, oracle_mod, e4m3_table, rows, a_cols, b_cols, seed):
    """FP4 token concatenation with the scales in the 128x4 tile layout: the
    scale bytes equal the oracle's row-major scales rearranged into tiles by
    the oracle (pad rows included), and every row's codes equal the oracle's."""
    _print_case("token_cat_fp4 128x4", rows, a_cols, b_cols, seed)
    inp = synth.token_cat_inputs(rows, a_cols, b_cols, seed=seed)
    cols, rows_pad = a_cols + b_cols, (rows + 127) // 128 * 128
    packed = Guarded((rows, cols // 2), torch.uint8)
    scales = Guarded((rows_pad, cols // 16), torch.uint8)
    qe.dit_token_cat_quant(qe.DIT_QUANT_FP4_E2M1_128X4, packed.t, scales.t, dev(inp.attn), a_cols,
                           dev(inp.mlp), b_cols, rows, dscalar(inp.fp4_g))
    torch.cuda.synchronize()
    packed.check("packed"), scales.check("scales")
    a_b, m_b = bits(inp.attn), bits(inp.mlp)
    ref_scales = np.zeros((rows_pad, cols // 16), np.uint8)

    def rows_scales(lo, hi):
        _, rs, _, _ = oracle_mod.token_cat_fp4(a_b[lo:hi], m_b[lo:hi], inp.fp4_g)
        ref_scales[lo:hi] = rs[:hi - lo]

    _parallel(rows_scales, rows)
    check_exact("128x4 scales", scales.bits().reshape(-1),
                oracle_mod.fp4_scales_to_128x4(ref_scales))
    # The codes: the tiled scale bytes equal the oracle's (above), so the
    # row-major comparison takes the oracle's scales as the GPU's.
    _check_fp4_rows(oracle_mod, e4m3_table, "fp4 128x4", packed.bits(), ref_scales, a_b, m_b,
                    inp.fp4_g)
    print("exact: codes 1.000000 scales 1.000000")


def test_token_cat_fp4_all_bf16_values_unit_scale(qe, oracle_mod):
    """Every bf16 value in [-6, 6] through the FP4 path at unit scale: each
    16-element group holds +-6 (so amax / 6 * g = 1 with g = 1, the scale code
    is 0x38 and the element scale is exactly 1) and 15 test values, so every
    code is the E2M1 rounding of a bf16 value itself."""
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    pats = pats[(pats & 0x7FFF) <= 0x40C0]  # |x| <= 6, including -0 and subnormals
    pats = np.concatenate([pats, np.zeros((-pats.size) % 15, np.uint16)]).reshape(-1, 15)
    anchor = np.where(np.arange(pats.shape[0]) % 2 == 0, 0x40C0, 0xC0C0).astype(np.uint16)
    groups = np.concatenate([anchor[:, None], pats], axis=1)  # [n_groups, 16]
    groups = np.concatenate([groups, np.tile(groups[:1], ((-groups.shape[0]) % 64, 1))])
    rows_bits = groups.reshape(-1, 64 * 16)  # 1024 columns per row
    rows = rows_bits.shape[0]
    a = torch.from_numpy(rows_bits.view(np.int16)).view(torch.bfloat16)
    packed, scales = qe.token_cat_quant(qe.DIT_QUANT_FP4_E2M1, dev(a), None, dscalar(1.0))
    rp, rs, _, _ = oracle_mod.token_cat_fp4(rows_bits, np.zeros((rows, 0), np.uint16), 1.0)
    gs = scales.cpu().numpy()
    assert np.all(gs[:rows] == 0x38) and np.all(gs[rows:] == 0)
    assert np.all(rs[:rows] == 0x38) and np.all(rs[rows:] == 0)
    check_exact("codes", packed.cpu().numpy(), rp)
    # The codes are the E2M1 rounding of each value itself.
    x = oracle_mod.f32_from_bf16(rows_bits)
    want = oracle_mod.e2m1_encode(x)
    got = packed.cpu().numpy()
    nib = np.stack([got & 0xF, got >> 4], axis=-1).reshape(rows, -1)
    same = (nib == want) | (((nib | want) & 7) == 0)  # +0 and -0 both encode zero
    assert same.all()


# ---------------------------------------------------------------------------
# Boundary behaviour on the device
# ---------------------------------------------------------------------------

def test_zero_rows_and_refusals_leave_outputs_untouched(qe):
    y = Guarded((4, 3072), torch.bfloat16)
    q = Guarded((4, 3072), torch.uint8)
    x = torch.randn(4, 3072, device="cuda").to(torch.bfloat16)
    sc = torch.zeros(3072, device="cuda", dtype=torch.bfloat16)
    s = dscalar(0.0625)
    before = y.buf.clone(), q.buf.clone()
    qe.dit_norm_modulate_fp8(y.t, q.t, x, sc, sc, s, 0, 3072, 1e-6)  # rows == 0: no-op
    with pytest.raises(qe.DitError) as e:  # 2-byte offset: refused
        qe.dit_norm_modulate_fp8(y.t, q.t, x.view(-1)[1:].data_ptr(), sc, sc, s, 3, 3072, 1e-6)
    assert e.value.status == qe.DIT_ERR_ALIGN
    with pytest.raises(qe.DitError) as e:
        qe.dit_norm_modulate_fp8(y.t, q.t, x, sc, sc, s, 4, 3076, 1e-6)
    assert e.value.status == qe.DIT_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert torch.equal(y.buf, before[0]) and torch.equal(q.buf, before[1])


def test_runs_on_a_side_stream(qe):
    inp = synth.bias_mul_add_inputs(64, 3072, seed=12)
    x, b, g, r = dev(inp.x), dev(inp.bias), dev(inp.gate), dev(inp.residual)
    ref = qe.bias_mul_add(x, b, g, r)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        out = qe.bias_mul_add(x, b, g, r)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert torch.equal(ref, out)


def test_hip_graph_capture_replays_match_eager(qe):
    """Every entry point is recorded into one HIP graph (through torch's graph
    capture on the current stream) and replayed three times, with eager work
    that overwrites the outputs in between; each replay must reproduce the
    eager results bit for bit."""
    torch.manual_seed(3)
    H, R = 3072, 256
    x = torch.randn(R, H, device="cuda").to(torch.bfloat16)
    res = torch.randn(R, H, device="cuda").to(torch.bfloat16)
    vec = lambda std, mean=0.0: (torch.randn(H, device="cuda") * std + mean).to(torch.bfloat16)
    sc, sh, bias, gate = vec(0.1), vec(0.1), vec(0.02), vec(0.1, 1.0)
    s8, g4 = dscalar(0.0625), dscalar(448.0)
    inp = synth.qkv_inputs(64, 16, 24, 128, seed=4)
    qkv_img, qkv_txt = dev(inp.img_qkv), dev(inp.txt_qkv)
    W = inp.width
    tabs = [torch.from_numpy(np.ascontiguousarray(t)).cuda()
            for t in (inp.img_cos, inp.img_sin, inp.txt_cos, inp.txt_sin)]
    ws = [dev(w) for w in (inp.img_q_w, inp.img_k_w, inp.txt_q_w, inp.txt_k_w)]
    a, m = x[:, :1024].contiguous(), x[:, 1024:].contiguous()

    outs = {
        "y": torch.empty(R, H, dtype=torch.bfloat16, device="cuda"),
        "dy": torch.empty(R, H, dtype=torch.bfloat16, device="cuda"),
        "dq": torch.empty(R, H, dtype=torch.uint8, device="cuda"),
        "dy2": torch.empty(R // 2, H, dtype=torch.bfloat16, device="cuda"),
        "dq2": torch.empty(R // 2, H, dtype=torch.uint8, device="cuda"),
        "q": torch.empty(R, H, dtype=torch.uint8, device="cuda"),
        "r": torch.empty(R, H, dtype=torch.bfloat16, device="cuda"),
        "y2": torch.empty(R, H, dtype=torch.bfloat16, device="cuda"),
        "q2": torch.empty(R, H, dtype=torch.uint8, device="cuda"),
        "r4": torch.empty(R, H, dtype=torch.bfloat16, device="cuda"),
        "p4": torch.empty(R, H // 2, dtype=torch.uint8, device="cuda"),
        "s4": torch.empty(R, H // 16, dtype=torch.uint8, device="cuda"),
        "jq": torch.empty(80, 24, 128, dtype=torch.bfloat16, device="cuda"),
        "jk": torch.empty(80, 24, 128, dtype=torch.bfloat16, device="cuda"),
        "jv": torch.empty(80, 24, 128, dtype=torch.bfloat16, device="cuda"),
        "bma": torch.empty(R, H, dtype=torch.bfloat16, device="cuda"),
        "c8": torch.empty(R, H, dtype=torch.uint8, device="cuda"),
        "c4": torch.empty(R, H // 2, dtype=torch.uint8, device="cuda"),
        "c4s": torch.empty(R, H // 16, dtype=torch.uint8, device="cuda"),
    }

    def run():
        o = outs
        qe.dit_norm_modulate_fp8(o["y"], o["q"], x, sc, sh, s8, R, H, 1e-6)
        qe.dit_norm_modulate_fp8_dual(o["dy"], o["dq"], x, sc, sh, s8, R, 1e-6, o["dy2"], o["dq2"],
                                      res, sh, sc, g4, R // 2, 1e-5, H)
        qe.dit_scale_residual_norm_modulate_fp8(o["r"], o["y2"], o["q2"], x, bias, gate, res, sc,
                                                sh, s8, R, H, 1e-6)
        qe.dit_scale_residual_norm_modulate_fp4(o["r4"], None, o["p4"], o["s4"],
                                                qe.DIT_FP4_SCALES_128X4, x, bias, gate, res, sc,
                                                sh, g4, R, H, 1e-6)
        qe.dit_qkv_epilogue(o["jq"], o["jk"], o["jv"], qkv_img[:, :W], qkv_img[:, W:2 * W],
                            qkv_img[:, 2 * W:], 64, 3 * W, qkv_txt[:, :W], qkv_txt[:, W:2 * W],
                            qkv_txt[:, 2 * W:], 16, 3 * W, *ws, *tabs, 64, 24, 128, 1e-6, 1e-6)
        qe.dit_bias_mul_add(o["bma"], x, bias, gate, res, R, H)
        qe.dit_token_cat_quant(qe.DIT_QUANT_FP8_E4M3, o["c8"], None, a, 1024, m, H - 1024, R, s8)
        qe.dit_token_cat_quant(qe.DIT_QUANT_FP4_E2M1, o["c4"], o["c4s"], a, 1024, m, H - 1024,
                               R, g4)

    run()
    torch.cuda.synchronize()
    eager = {k: v.clone() for k, v in outs.items()}
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    torch.cuda.synchronize()
    for rep in range(3):
        for v in outs.values():  # eager work between replays
            v.view(torch.uint8).fill_(0xA5 + rep)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, v in outs.items():
            assert torch.equal(v.view(torch.uint8), eager[k].view(torch.uint8)), (rep, k)


def _bf16_band(rng, shape, exp_lo, exp_hi, sign=None):
    """Random bf16 bit patterns with biased exponents in [exp_lo, exp_hi)."""
    sign = rng.integers(0, 2, shape) if sign is None else sign
    exp = rng.integers(exp_lo, exp_hi, shape)
    man = rng.integers(0, 128, shape)
    return ((sign << 15) | (exp << 7) | man).astype(np.uint16)


@pytest.mark.parametrize("band", ["top", "bottom"])
def test_fma_products_at_fp32_range_edges(qe, oracle_mod, e4m3_table, band):
    """The single-rounded x * gate + residual at the edges of the products'
    supported range (|x gate| < 2^128, where the fp32 product is exact):
    products in [2^127, 1.72 * 2^127) against residuals of opposite sign near
    the bf16 maximum (large cancellations, every result finite), and products
    so small that fp32 underflows against zero or subnormal residuals. Both
    bias_mul_add and the gated residual of the norm must reproduce the
    oracle's exact rounding bit for bit; at the bottom only the sign of a zero
    may differ (the library documents that a product fp32 cannot hold keeps
    only its sign)."""
    _print_case("fma at fp32 range edges", band)
    rng = np.random.default_rng(11 if band == "top" else 12)
    R, H = 4, 3072
    if band == "top":
        # unbiased factor exponents summing to 127, significands below 1.32
        ge = rng.integers(188, 194, H)
        gb = ((rng.integers(0, 2, H) << 15) | (ge << 7) | rng.integers(0, 41, H)).astype(np.uint16)
        xs = rng.integers(0, 2, (R, H))
        xb = ((xs << 15) | ((381 - ge)[None, :] << 7) | rng.integers(0, 41, (R, H))).astype(np.uint16)
        prod_sign = (xs ^ (gb[None, :] >> 15)).astype(np.int64)
        rb = (((1 - prod_sign) << 15) | (254 << 7) | rng.integers(0, 128, (R, H))).astype(np.uint16)
    else:
        xb = _bf16_band(rng, (R, H), 50, 66)
        gb = _bf16_band(rng, (H,), 50, 66)
        rb = _bf16_band(rng, (R, H), 0, 2)
        rb[:, ::2] = 0  # half the residuals +0: the sum is the product alone
    t = lambda b: dev(torch.from_numpy(b.view(np.int16)).view(torch.bfloat16))
    u16 = lambda g: g.cpu().view(torch.int16).numpy().view(np.uint16)

    def same(name, gpu, ref):
        if band == "bottom":  # +-0 compare equal
            zero = ((gpu & 0x7FFF) == 0) & ((ref & 0x7FFF) == 0)
            gpu, ref = np.where(zero, 0, gpu), np.where(zero, 0, ref)
        check_exact(name, gpu, ref)

    y = qe.bias_mul_add(t(xb), None, t(gb), t(rb))
    same("bias_mul_add", u16(y), oracle_mod.bias_mul_add(xb, None, gb, rb))

    scale = synth.bf16_bits((torch.randn(H, generator=torch.Generator().manual_seed(5)) * 0.1)
                            .to(torch.bfloat16))
    shift = synth.bf16_bits((torch.randn(H, generator=torch.Generator().manual_seed(6)) * 0.1)
                            .to(torch.bfloat16))
    r, yy, q = qe.scale_residual_norm_modulate_fp8(t(xb), None, t(gb), t(rb), t(scale), t(shift),
                                                   dscalar(0.0625), 1e-6)
    rr, ryy, rq, pre = oracle_mod.scale_residual_norm_modulate_fp8(
        xb, None, gb, rb, scale, shift, float(np.float32(0.0625)), 1e-6)
    assert np.isfinite(oracle_mod.f32_from_bf16(rr)).all()
    same("residual_out", u16(r), rr)
    check_bf16("y", u16(yy), ryy)
    check_fp8("q", q.cpu().numpy(), rq, pre, e4m3_table)


@pytest.mark.parametrize("g", [1.0, 2.0 ** -60, 2.0 ** -120, 2.0 ** 60])
def test_fp4_group_scale_for_every_bf16_maximum(qe, oracle_mod, e4m3_table, g):
    """Every finite non-negative bf16 value as a 16-element group's maximum
    (one group per value, the rest of the group zero; signs alternate), under
    global scales that bring small and huge maxima into the unclamped range of
    the E4M3 group scale: the scale bytes, which depend on amax / 6 rounded
    once, must equal the oracle's exactly, and the codes within the FP4 rule."""
    _print_case("fp4 group scale, every bf16 maximum", g)
    n = 0x7F80  # +0 .. the largest finite bf16
    cols = 256  # 16 groups per row
    rows = -(-n // (cols // 16))
    x = np.zeros((rows, cols), np.uint16)
    amax = np.arange(rows * (cols // 16), dtype=np.int64) % n
    sign = (np.arange(rows * (cols // 16)) % 2).astype(np.uint16) << 15
    x.reshape(-1, 16)[:, 0] = amax.astype(np.uint16) | sign
    x.reshape(-1, 16)[:, 7] = (amax // 2).astype(np.uint16)  # a smaller second value
    t = dev(torch.from_numpy(x.view(np.int16)).view(torch.bfloat16))
    packed, scales = qe.token_cat_quant(qe.DIT_QUANT_FP4_E2M1, t, None, dscalar(g))
    rp, rs, s_pre, pre = oracle_mod.token_cat_fp4(x, np.zeros((rows, 0), np.uint16), g)
    check_exact("scales", scales.cpu().numpy(), rs)
    check_fp4("fp4", packed.cpu().numpy(), scales.cpu().numpy(), rp, rs, s_pre, pre,
              oracle_mod.f32_from_bf16(x), g, e4m3_table, oracle_mod.e2m1_encode)


def test_degenerate_inputs(qe, oracle_mod, e4m3_table):
    """Constant, zero and outlier rows through the norms (with FP8 saturation
    and NVFP4), zero and huge heads through the QKV epilogue, and all-zero,
    single-value and subnormal groups through the FP4 token concatenation."""
    H = 3072
    rows = np.zeros((8, H), np.float32)
    rows[0] = 2.5                               # constant: variance 0
    rows[2, 17] = 1e30                          # one outlier
    rows[3] = np.where(np.arange(H) % 2, 1e-30, -1e-30)  # tiny alternating
    rows[4] = np.linspace(-40000, 40000, H)     # wide range
    rows[5, ::7] = 3.0                          # sparse
    rows[6] = 1e-38                             # near the smallest normal
    rows[7] = -7.0                              # negative constant
    x = torch.from_numpy(rows).to(torch.bfloat16)
    sc = torch.from_numpy(np.random.default_rng(0).standard_normal(H).astype(np.float32) * 0.1).to(torch.bfloat16)
    sh = torch.from_numpy(np.random.default_rng(1).standard_normal(H).astype(np.float32) * 0.1).to(torch.bfloat16)
    for input_scale in (1e-3, 0.0625):          # 1e-3: most FP8 codes saturate
        y, q = qe.norm_modulate_fp8(dev(x), dev(sc), dev(sh), dscalar(input_scale), 1e-6)
        ry, rq, pre = oracle_mod.norm_modulate_fp8(bits(x), bits(sc), bits(sh),
                                                   float(np.float32(input_scale)), 1e-6)
        check_bf16("degenerate y", y.cpu().view(torch.int16).numpy().view(np.uint16), ry)
        check_fp8("degenerate q", q.cpu().numpy(), rq, pre, e4m3_table)
    y4, p4, s4 = qe.norm_modulate_fp4(dev(x), dev(sc), dev(sh), dscalar(448.0), 1e-6)
    ry, rp, rs, s_pre, pre = oracle_mod.norm_modulate_fp4(bits(x), bits(sc), bits(sh), 448.0, 1e-6)
    check_bf16("degenerate fp4 y", y4.cpu().view(torch.int16).numpy().view(np.uint16), ry)
    check_fp4("degenerate fp4", p4.cpu().numpy(), s4.cpu().numpy(), rp, rs, s_pre, pre,
              oracle_mod.f32_from_bf16(ry), 448.0, e4m3_table, oracle_mod.e2m1_encode)

    # QKV: head 0 of every token all zero (mean square 0), head 1 huge.
    inp = synth.qkv_inputs(6, 2, 4, 128, seed=7)
    for packed in (inp.img_qkv, inp.txt_qkv):
        v = packed.float()
        v[:, 0:128] = 0.0
        v[:, 128:256] *= 1e30
        v[:, 512:640] = 0.0        # K head 0
        packed.copy_(v.to(torch.bfloat16))
    gq, gk, gv = _run_qkv(qe, inp)
    rq, rk, rv = _oracle_qkv(oracle_mod, inp)
    check_bf16("degenerate joint_q", gq, rq)
    check_bf16("degenerate joint_k", gk, rk)
    check_exact("degenerate joint_v", gv, rv)

    # FP4 groups: all zero, one non-zero value, subnormal bf16 values.
    cols = 64
    g = np.zeros((4, cols), np.float32)
    g[0, 16 + 5] = -3.0
    g[1, :16] = 1e-39                       # bf16 subnormals
    g[2, 32:48] = np.arange(16) * 0.25
    g[3] = 6.0
    gb = torch.from_numpy(g).to(torch.bfloat16)
    for gv_ in (1.0, 448.0):
        pk, scs = qe.token_cat_quant(qe.DIT_QUANT_FP4_E2M1, dev(gb), None, dscalar(gv_))
        rp, rs, s_pre, pre = oracle_mod.token_cat_fp4(bits(gb), np.zeros((4, 0), np.uint16), gv_)
        check_fp4("degenerate groups", pk.cpu().numpy(), scs.cpu().numpy(), rp, rs, s_pre, pre,
                  oracle_mod.f32_from_bf16(bits(gb)), gv_, e4m3_table, oracle_mod.e2m1_encode)

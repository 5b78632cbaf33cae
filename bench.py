"""Benchmark of the fused DiT-block epilogues on one MI355X.

One step = one pass over every fused epilogue at its full workload shape:
  norm_dual  dit_norm_modulate_fp8_dual            [4096, 3072] image + [512, 3072] text tokens
  qkv        dit_qkv_epilogue                      512 text + 4096 image tokens, 24 x 128
  sr_norm    dit_scale_residual_norm_modulate_fp8  [4096, 3072] with bias
  bma        dit_bias_mul_add                      [4608, 3072]
  cat_fp8    dit_token_cat_quant FP8               [4608, 6144 + 18432]
  cat_fp4    dit_token_cat_quant FP4               [4608, 6144 + 18432]
Inputs are seeded synthetic tensors already resident in HBM; every launch has
its own buffers, so one step touches 1.07 GB and no kernel finds its inputs
in the 256 MB Infinity Cache from the previous step.

Bytes are compulsory bytes: every input read once, every output written once,
row-broadcast vectors once. The printed JSON line reports the whole-step
throughput (GB/s) over exactly --steps timed steps, taken after --warmup
untimed steps and a settling phase that keeps the GPU busy until its step
time is steady (the spread of further timed windows is reported beside it);
per kernel, its mean duration launched back to back over rotating buffer sets
(us_per_call, GB/s); the roofline entry of the kernel that takes the most
time; and the CPU oracle timed on a row sample.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--blocks N]
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E peak, 8 TB/s
METRIC = "fused-epilogue HBM GB/s (% of MI355X peak) + µs/call at Qwen-Image shapes"

QWEN_HIDDEN, IMG, TXT, HEADS, HEAD_DIM = 3072, 4096, 512, 24, 128
FLUX_ROWS, FLUX_A, FLUX_B = 4608, 6144, 18432
FLUX_HEADS = 48  # FLUX.2: hidden 6144 = 48 heads x 128
NORM_ROWS = (127, 128, 1024)  # LN + FP8 row counts timed beside the step (4096 is in it)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---- compulsory bytes per launch ------------------------------------------------

def bytes_norm(rows, hidden, y=True, q=True):
    return (2 + 2 * y + q) * rows * hidden + 4 * hidden + 4 * q


def bytes_sr(rows, hidden, bias=True, y=True, q=True):
    return (6 + 2 * y + q) * rows * hidden + (8 if bias else 6) * hidden + 4 * q


def bytes_qkv(n_tok, heads, head_dim):
    return 12 * n_tok * heads * head_dim + 2 * 4 * n_tok * (head_dim // 2) + 4 * 2 * head_dim


def bytes_sr_fp4(rows, hidden, bias=True, y=True):
    rows_pad = (rows + 127) // 128 * 128
    return ((6 + 2 * y) * rows * hidden + rows * hidden // 2 + rows_pad * (hidden // 16)
            + (8 if bias else 6) * hidden + 4)


def bytes_bma(rows, hidden, bias=True):
    return 6 * rows * hidden + (4 if bias else 2) * hidden


def bytes_cat_fp8(rows, cols):
    return 3 * rows * cols + 4


def bytes_cat_fp4(rows, cols):
    return 2 * rows * cols + rows * cols // 2 + (rows + 127) // 128 * 128 * (cols // 16) + 4


# ---- workload ---------------------------------------------------------------------

class Workload:
    """Device buffers and the launch list of one step. `names` selects launches."""

    ALL = ("norm_dual", "qkv", "sr_norm", "bma", "cat_fp8", "cat_fp4")
    # Timed beside the step, not in it: the FLUX.2 shape of the QKV epilogue
    # (4096 image + 512 text tokens, 48 heads, one shared [cos | sin] cache),
    # the FP8-only LayerNorm + modulation at the FLUX.2 shape (4608 x 6144, no
    # bf16 output), the bf16-only bias + gated-residual norm (no FP8) and the
    # same norm with NVFP4 output (4096 x 3072, g = 448), and the FP4 token
    # concatenation writing its scales in the 128x4 tile layout.
    # The image and text norms of norm_dual as separate launches are timed
    # beside it too.
    EXTRA = ("qkv_flux2", "norm_flux2_fp8", "sr_norm_bf16", "sr_norm_fp4", "cat_fp4_128x4",
             "norm_img", "norm_txt")

    def __init__(self, torch, qe, seed=0, names=ALL):
        import numpy as np

        import synth

        dev = torch.device("cuda:0")
        g = torch.Generator(device=dev)
        g.manual_seed(seed)

        def randn(*shape, std=1.0, mean=0.0):
            return (torch.randn(*shape, generator=g, device=dev) * std + mean).to(torch.bfloat16)

        def empty(*shape, dtype=torch.bfloat16):
            return torch.empty(*shape, dtype=dtype, device=dev)

        def scalar(v):
            return torch.tensor([v], dtype=torch.float32, device=dev)

        H = QWEN_HIDDEN
        W = HEADS * HEAD_DIM
        C = FLUX_A + FLUX_B
        s0625 = scalar(0.0625)
        self.keep = []  # keeps every buffer alive; launches take raw device addresses
        st = torch.cuda.current_stream(dev).cuda_stream

        def P(*ts):
            self.keep.extend(ts)
            return [None if t is None else t.data_ptr() for t in ts]

        def norm(rows, hidden=H, want_y=True):
            x, sc, sh = randn(rows, hidden), randn(hidden, std=0.1), randn(hidden, std=0.1)
            y = empty(rows, hidden) if want_y else None
            q = empty(rows, hidden, dtype=torch.uint8)
            p = P(y, q, x, sc, sh, s0625)
            return bytes_norm(rows, hidden, y=want_y), lambda: qe.dit_norm_modulate_fp8(
                *p, rows, hidden, 1e-6, stream=st)

        def norm_dual():
            xi, sci, shi = randn(IMG, H), randn(H, std=0.1), randn(H, std=0.1)
            xt, sct, sht = randn(TXT, H), randn(H, std=0.1), randn(H, std=0.1)
            yi, qi = empty(IMG, H), empty(IMG, H, dtype=torch.uint8)
            yt, qt = empty(TXT, H), empty(TXT, H, dtype=torch.uint8)
            pi = P(yi, qi, xi, sci, shi, s0625)
            pt = P(yt, qt, xt, sct, sht, scalar(0.02))
            return bytes_norm(IMG, H) + bytes_norm(TXT, H), lambda: qe.dit_norm_modulate_fp8_dual(
                *pi, IMG, 1e-6, *pt, TXT, 1e-6, H, stream=st)

        def qkv(heads=HEADS, shared_cache=False):
            W = heads * HEAD_DIM
            img, txt = randn(IMG, 3 * W), randn(TXT, 3 * W)
            ws = [randn(HEAD_DIM, std=0.05, mean=1.0) for _ in range(4)]
            tc, ts = synth.rope_tables(np.arange(TXT), HEAD_DIM)
            ic, is_ = synth.rope_tables(np.arange(TXT, TXT + IMG), HEAD_DIM)
            half = HEAD_DIM // 2
            if shared_cache:  # one [txt + img, 128] cache, rows [cos | sin] in joint order
                cache = torch.from_numpy(np.concatenate(
                    [np.concatenate([tc, ts], 1), np.concatenate([ic, is_], 1)])).to(dev)
                tables, stride = (cache[TXT:, :half], cache[TXT:, half:], cache[:TXT, :half],
                                  cache[:TXT, half:]), 2 * half
            else:
                tables, stride = tuple(torch.from_numpy(a).to(dev) for a in (ic, is_, tc, ts)), half
            jq, jk, jv = (empty(IMG + TXT, heads, HEAD_DIM) for _ in range(3))
            o = P(jq, jk, jv)
            i3 = P(img[:, :W], img[:, W:2 * W], img[:, 2 * W:])
            t3 = P(txt[:, :W], txt[:, W:2 * W], txt[:, 2 * W:])
            w4 = P(*ws)
            r4 = P(*tables)
            return bytes_qkv(IMG + TXT, heads, HEAD_DIM), lambda: qe.dit_qkv_epilogue(
                *o, *i3, IMG, 3 * W, *t3, TXT, 3 * W, *w4, *r4, stride, heads, HEAD_DIM,
                1e-6, 1e-6, stream=st)

        def sr_norm(want_q=True):
            x, res = randn(IMG, H), randn(IMG, H)
            b, gt = randn(H, std=0.02), randn(H, std=0.1, mean=1.0)
            sc, sh = randn(H, std=0.1), randn(H, std=0.1)
            r, y = empty(IMG, H), empty(IMG, H)
            q = empty(IMG, H, dtype=torch.uint8) if want_q else None
            p = P(r, y, q, x, b, gt, res, sc, sh, s0625 if want_q else None)
            return bytes_sr(IMG, H, q=want_q), lambda: qe.dit_scale_residual_norm_modulate_fp8(
                *p, IMG, H, 1e-6, stream=st)

        def sr_norm_fp4():
            x, res = randn(IMG, H), randn(IMG, H)
            b, gt = randn(H, std=0.02), randn(H, std=0.1, mean=1.0)
            sc, sh = randn(H, std=0.1), randn(H, std=0.1)
            r, y = empty(IMG, H), empty(IMG, H)
            packed = empty(IMG, H // 2, dtype=torch.uint8)
            scales = empty((IMG + 127) // 128 * 128, H // 16, dtype=torch.uint8)
            p = P(r, y, packed, scales, x, b, gt, res, sc, sh, scalar(448.0))
            return bytes_sr_fp4(IMG, H), lambda: qe.dit_scale_residual_norm_modulate_fp4(
                *p[:4], qe.DIT_FP4_SCALES_ROW_MAJOR, *p[4:], IMG, H, 1e-6, stream=st)

        def bma():
            R = IMG + TXT
            x, res = randn(R, H), randn(R, H)
            b, gt = randn(H, std=0.02), randn(H, std=0.5)
            y = empty(R, H)
            p = P(y, x, b, gt, res)
            return bytes_bma(R, H), lambda: qe.dit_bias_mul_add(*p, R, H, stream=st)

        def cat(kind):
            a, m = randn(FLUX_ROWS, FLUX_A), randn(FLUX_ROWS, FLUX_B)
            if kind == qe.DIT_QUANT_FP8_E4M3:
                out, scales, s = empty(FLUX_ROWS, C, dtype=torch.uint8), None, scalar(0.05)
                nbytes = bytes_cat_fp8(FLUX_ROWS, C)
            else:
                out = empty(FLUX_ROWS, C // 2, dtype=torch.uint8)
                scales = empty((FLUX_ROWS + 127) // 128 * 128, C // 16, dtype=torch.uint8)
                amax = max(float(a.float().abs().max()), float(m.float().abs().max()))
                s = scalar(float(np.float32(np.float32(2688.0) / np.float32(amax))))
                nbytes = bytes_cat_fp4(FLUX_ROWS, C)
            po, ps, pa, pm, pscale = P(out, scales, a, m, s)
            return nbytes, lambda: qe.dit_token_cat_quant(kind, po, ps, pa, FLUX_A, pm, FLUX_B,
                                                          FLUX_ROWS, pscale, stream=st)

        builders = {
            "norm_dual": norm_dual,
            "norm_img": lambda: norm(IMG), "norm_txt": lambda: norm(TXT), "qkv": qkv,
            "sr_norm": sr_norm, "bma": bma,
            "cat_fp8": lambda: cat(qe.DIT_QUANT_FP8_E4M3),
            "cat_fp4": lambda: cat(qe.DIT_QUANT_FP4_E2M1),
            "qkv_flux2": lambda: qkv(heads=FLUX_HEADS, shared_cache=True),
            "norm_flux2_fp8": lambda: norm(FLUX_ROWS, FLUX_A, want_y=False),
            "sr_norm_bf16": lambda: sr_norm(want_q=False),
            "sr_norm_fp4": sr_norm_fp4,
            "cat_fp4_128x4": lambda: cat(qe.DIT_QUANT_FP4_E2M1_128X4),
        }
        for r in NORM_ROWS:  # the plain norm at other row counts
            builders["norm_r%d" % r] = lambda r=r: norm(r)
        self.launches = []  # (name, compulsory bytes, launch)
        for n in names:
            nbytes, fn = builders[n]()
            self.launches.append((n, nbytes, fn))
        self.step_bytes = sum(b for _, b, _ in self.launches)

    def step(self):
        for _, _, fn in self.launches:
            fn()


def time_launches(torch, fns, reps):
    """Mean time of `reps` launches issued back to back on torch's current
    stream (where the kernels run), cycling through `fns`, between two events
    recorded on that stream; plus the host wall time of the same region."""
    stream = torch.cuda.current_stream()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(reps):
        fns[i % len(fns)]()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return start.elapsed_time(end) / reps, wall / reps


def time_steps(torch, wl, steps):
    """Mean ms per step (all launches of `wl`, in order)."""
    fns = [fn for _, _, fn in wl.launches]

    def step():
        for fn in fns:
            fn()

    return time_launches(torch, [step], steps)


ROTATION_BYTES = 640 << 20  # > 2x the 256 MB Infinity Cache


SETTLE_S = 0.5       # untimed GPU work before the timed steps
SETTLE_STEP_TOL = 0.01  # ... until two consecutive 20-step windows agree within 1%
SPREAD_WINDOWS = 5   # timed windows of --steps steps each, after the headline one


def settle(torch, wl):
    """Untimed steps until the GPU has run the step for at least SETTLE_S
    seconds and two consecutive 20-step windows agree within 1% (at most 4 s):
    the timed steps then run at steady clocks. Returns the steps run and the
    ms per step of the first 8 and the last 2 windows (the warm-up ramp)."""
    n, t0, prev, trace = 0, time.perf_counter(), None, []
    while True:
        ms, _ = time_steps(torch, wl, 20)
        trace.append(round(ms, 4))
        n += 20
        elapsed = time.perf_counter() - t0
        steady = prev is not None and abs(ms - prev) <= SETTLE_STEP_TOL * prev
        if (elapsed >= SETTLE_S and steady) or elapsed >= 4.0:
            return n, trace[:8] + (trace[-2:] if len(trace) > 10 else trace[8:])
        prev = ms


KERNEL_PASSES = 5


def kernel_timings(torch, qe, wl, steps):
    """Per launch: its mean duration when launched back to back, cycling
    through enough independent buffer sets that the sets together exceed
    twice the Infinity Cache (so every launch reads from HBM).

    Setting up the buffer sets leaves the GPU idle for a while, and the first
    launches after it run slower. So one pass of `reps` launches goes
    untimed; then KERNEL_PASSES passes are timed and their median is the
    figure (the passes are reported too)."""
    out = {}
    for name, nbytes, fn in wl.launches:
        # The extra Workload objects own the buffers their launches address:
        # they stay referenced until the timing below has synchronised.
        extra = [Workload(torch, qe, seed=1000 + i, names=(name,))
                 for i in range(1, -(-ROTATION_BYTES // nbytes))]
        sets = [fn] + [w.launches[0][2] for w in extra]
        reps = max(100, 2 * len(sets))
        for f in sets:
            f()
        time_launches(torch, sets, reps)
        passes = [time_launches(torch, sets, reps)[0] for _ in range(KERNEL_PASSES)]
        out[name] = {"iso_ms": statistics.median(passes), "passes_ms": passes,
                     "sets": len(sets), "reps": reps}
        del sets, extra
    return out


def pass_range_us(t):
    """The fastest and slowest timed pass of a launch, in us."""
    return [round(1e3 * min(t["passes_ms"]), 3), round(1e3 * max(t["passes_ms"]), 3)]


# Source files that define each launch's kernel (for matching profiled traffic).
KERNEL_SOURCES = {
    "norm_dual": "norm_modulate.hip", "norm_img": "norm_modulate.hip",
    "norm_txt": "norm_modulate.hip", "sr_norm": "norm_modulate.hip",
    "qkv": "qkv_epilogue.hip", "bma": "bias_mul_add.hip", "cat_fp8": "token_cat_quant.hip",
    "cat_fp4": "token_cat_quant.hip", "qkv_flux2": "qkv_epilogue.hip",
    "norm_flux2_fp8": "norm_modulate.hip", "sr_norm_bf16": "norm_modulate.hip",
    "sr_norm_fp4": "norm_modulate.hip", "cat_fp4_128x4": "token_cat_quant.hip",
}


def kernel_source_hash(name):
    """sha256 over the kernel's source file and the shared device headers."""
    import hashlib

    csrc = os.path.join(ROOT, "quant_epilogues_amd", "csrc")
    h = hashlib.sha256()
    for f in (KERNEL_SOURCES[name], "dit_device.h", "kernels.h"):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def profiled_traffic(name):
    """HBM bytes per launch measured with rocprofv3 FETCH_SIZE / WRITE_SIZE
    (scaled by a plain-copy calibration), from the committed summary in
    profiles/; None if absent or if the kernel source changed since."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic_qwen_flux_step.md")
    try:
        with open(path) as f:
            text = f.read()
        block = text.split("```json", 1)[1].split("```", 1)[0]
        rec = json.loads(block)["launches"][name]
    except (OSError, IndexError, KeyError, ValueError):
        return None
    if rec.get("source_sha256") != kernel_source_hash(name):
        return None
    return rec["hbm_bytes"]


def cpu_threads():
    """Host threads for the all-core oracle run: the cores this process may
    use, at most 16 (a one-GPU share of the GPU host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_model() -> str:
    """The host CPU's model name, from /proc/cpuinfo."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(sample_div=2, threads=1):
    """The CPU oracle on a row sample of the same step: single-threaded, or
    (threads > 1) with every epilogue's rows cut into `threads` slices that
    run on a thread pool. The oracle is called as it stands; its C entry
    points release the GIL, so the slices run in parallel."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    import oracle
    import synth

    if not os.path.exists(oracle._LIB_PATH):
        oracle.build()
    H = QWEN_HIDDEN
    img, txt, flux = IMG // sample_div, TXT // sample_div, FLUX_ROWS // sample_div
    b = synth.bf16_bits
    nm_i = synth.norm_modulate_inputs(img, H, seed=0)
    nm_t = synth.norm_modulate_inputs(txt, H, seed=1)
    qk = synth.qkv_inputs(img, txt, HEADS, HEAD_DIM, seed=2)
    sr = synth.scale_residual_inputs(img, H, seed=3)
    bm = synth.bias_mul_add_inputs(img + txt, H, seed=4)
    tc = synth.token_cat_inputs(flux, FLUX_A, FLUX_B, seed=5)
    x_i, x_t = b(nm_i.x), b(nm_t.x)
    qi, qt = b(qk.img_qkv), b(qk.txt_qkv)
    qw = (b(qk.img_q_w), b(qk.img_k_w), b(qk.txt_q_w), b(qk.txt_k_w))
    srx, srr = b(sr.x), b(sr.residual)
    bmx, bmr = b(bm.x), b(bm.residual)
    ta, tm = b(tc.attn), b(tc.mlp)

    def cuts(n):  # `threads` contiguous row ranges covering [0, n)
        return [(n * k // threads, n * (k + 1) // threads) for k in range(threads)]

    tasks = []
    for lo, hi in cuts(img):
        tasks.append(lambda lo=lo, hi=hi: oracle.norm_modulate_fp8(
            x_i[lo:hi], b(nm_i.scale), b(nm_i.shift), 0.0625, 1e-6))
        tasks.append(lambda lo=lo, hi=hi: oracle.scale_residual_norm_modulate_fp8(
            srx[lo:hi], b(sr.bias), b(sr.gate), srr[lo:hi], b(sr.scale), b(sr.shift), 0.0625, 1e-6))
    for lo, hi in cuts(txt):
        tasks.append(lambda lo=lo, hi=hi: oracle.norm_modulate_fp8(
            x_t[lo:hi], b(nm_t.scale), b(nm_t.shift), 0.0625, 1e-6))
    for (ilo, ihi), (tlo, thi) in zip(cuts(img), cuts(txt)):
        tasks.append(lambda ilo=ilo, ihi=ihi, tlo=tlo, thi=thi: oracle.qkv_epilogue_packed(
            qi[ilo:ihi], qt[tlo:thi], *qw, qk.img_cos[ilo:ihi], qk.img_sin[ilo:ihi],
            qk.txt_cos[tlo:thi], qk.txt_sin[tlo:thi], HEADS, HEAD_DIM, 1e-6, 1e-6))
    for lo, hi in cuts(img + txt):
        tasks.append(lambda lo=lo, hi=hi: oracle.bias_mul_add(
            bmx[lo:hi], b(bm.bias), b(bm.gate), bmr[lo:hi]))
    for lo, hi in cuts(flux):
        tasks.append(lambda lo=lo, hi=hi: oracle.token_cat_fp8(ta[lo:hi], tm[lo:hi], 0.05))
        tasks.append(lambda lo=lo, hi=hi: oracle.token_cat_fp4(ta[lo:hi], tm[lo:hi], tc.fp4_g))
    t0 = time.perf_counter()
    if threads == 1:
        for f in tasks:
            f()
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(lambda f: f(), tasks))
    secs = time.perf_counter() - t0
    C = FLUX_A + FLUX_B
    nbytes = (bytes_norm(img, H) + bytes_norm(txt, H) + bytes_qkv(img + txt, HEADS, HEAD_DIM)
              + bytes_sr(img, H) + bytes_bma(img + txt, H) + bytes_cat_fp8(flux, C)
              + bytes_cat_fp4(flux, C))
    how = "single thread" if threads == 1 else f"{threads} threads, rows cut into {threads} slices"
    return {"value": round(nbytes / secs / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"every epilogue of the step on 1/{sample_div} of its rows "
                      f"({img} image + {txt} text tokens, {flux} FLUX.2 rows), {how}, {secs:.1f} s"}


BLOCK_LAUNCHES = ("norm_dual", "qkv", "bma")


def block_sequence(torch, qe, blocks, reps):
    """Qwen-Image-shaped block sequence: per block the LayerNorm + modulation +
    FP8 of the image and text rows (one launch), the QKV epilogue and
    bias_mul_add, each block on its own random buffers."""
    wls = [Workload(torch, qe, seed=100 + i, names=BLOCK_LAUNCHES) for i in range(blocks)]
    for _ in range(2):  # untimed: the GPU idled while the buffers were set up
        for wl in wls:
            wl.step()
    torch.cuda.synchronize()
    events = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    events[0].record()
    for i in range(reps):
        for wl in wls:
            wl.step()
        events[i + 1].record()
    torch.cuda.synchronize()
    passes = [events[i].elapsed_time(events[i + 1]) for i in range(reps)]
    ms = statistics.median(passes)
    nbytes = sum(wl.step_bytes for wl in wls)
    return {"blocks": blocks, "launches": len(BLOCK_LAUNCHES) * blocks, "bytes": nbytes,
            "ms_per_pass": round(ms, 4), "ms_passes": [round(min(passes), 4), round(max(passes), 4)],
            "gb_s": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "pct_peak": round(100 * nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2)}


def copy_calibration(torch, nbytes=1 << 30, reps=5):
    """A plain device copy of known size, for scaling the FETCH_SIZE /
    WRITE_SIZE counters (each copy reads and writes `nbytes`)."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0").random_()
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_each_way": nbytes, "copies": reps}), flush=True)


def graph_us_per_call(torch, qe, name, nbytes, warm=False):
    """Mean GPU time per launch of `name` with no host launch cost in the
    way: the launches (cycling through rotating buffer sets whose total
    exceeds twice the Infinity Cache, or one set if `warm`) are captured
    once into a HIP graph on a side stream and the graph is replayed."""
    s = torch.cuda.Stream()
    nsets = 1 if warm else -(-ROTATION_BYTES // nbytes)
    with torch.cuda.stream(s):  # the launches bind the stream current at construction
        sets = [Workload(torch, qe, seed=2000 + i, names=(name,)) for i in range(nsets)]
        fns = [w.launches[0][2] for w in sets]
        for f in fns:
            f()
    torch.cuda.synchronize()
    calls = max(200, 2 * nsets)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for i in range(calls):
            fns[i % nsets]()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(s):
        g.replay()  # untimed first replay
        start.record()
        for _ in range(3):
            g.replay()
        end.record()
    torch.cuda.synchronize()
    us = 1e3 * start.elapsed_time(end) / (3 * calls)
    del g, sets, fns
    return us


def norm_rows_timings(torch, qe, steps):
    """The plain LN + modulation + FP8 norm (hidden 3072, bf16 y and FP8 q) at
    127, 128 and 1024 rows: per call with rotating buffers (cold, as every
    other launch), and on one buffer set launched back to back (warm), the
    latency figure for the 127-row case."""
    wl = Workload(torch, qe, seed=0, names=tuple("norm_r%d" % r for r in NORM_ROWS))
    t = kernel_timings(torch, qe, wl, steps)
    out = {}
    for (name, nbytes, fn), rows in zip(wl.launches, NORM_ROWS):
        iso = t[name]["iso_ms"]
        warm, host = time_launches(torch, [fn], max(steps, 100))
        # host_us_per_call near warm_us_per_call: the loop is bound by the
        # launch calls; the graph-replayed figures are the kernel's own.
        graph = graph_us_per_call(torch, qe, name, nbytes)
        out[str(rows)] = {"us_per_call": round(1e3 * iso, 3), "warm_us_per_call": round(1e3 * warm, 3),
                          "host_us_per_call": round(1e6 * host, 3),
                          "graph_us_per_call": round(graph, 3),
                          "graph_warm_us_per_call": round(graph_us_per_call(torch, qe, name, nbytes, True), 3),
                          "bytes": nbytes, "gb_s": round(nbytes / (iso * 1e-3) / 1e9, 1),
                          "graph_gb_s": round(nbytes / (graph * 1e-6) / 1e9, 1),
                          "rotation_sets": t[name]["sets"]}
    return out


def split_path_timings(torch, steps):
    """The unfused equivalents written as plain PyTorch GPU ops (separate
    norm, modulation and quantisation kernels with materialised bf16
    intermediates), timed like the fused launches with rotating inputs. For
    context only: the library never runs them, and their results are not
    checked. FP4 has no plain PyTorch form and is left out."""
    import torch.nn.functional as F

    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    bf16, fp8 = torch.bfloat16, torch.float8_e4m3fn
    H, W = QWEN_HIDDEN, HEADS * HEAD_DIM

    def randn(*shape, std=1.0, mean=0.0):
        return (torch.randn(*shape, generator=g, device=dev) * std + mean).to(bf16)

    def quant(y, inv):
        return (y.float() * inv).clamp_(-448.0, 448.0).to(fp8)

    def mk_norm():
        x, sc, sh = randn(IMG, H), randn(H, std=0.1), randn(H, std=0.1)
        return lambda: quant(F.layer_norm(x, (H,), eps=1e-6) * (1 + sc) + sh, 16.0)

    def mk_sr():
        x, res = randn(IMG, H), randn(IMG, H)
        b, gt, sc, sh = randn(H, std=0.02), randn(H, std=0.1, mean=1.0), randn(H, std=0.1), randn(H, std=0.1)

        def run():
            r = res + gt * (x + b)
            return r, quant(F.layer_norm(r, (H,), eps=1e-6) * (1 + sc) + sh, 16.0)
        return run

    def mk_qkv():
        img, txt = randn(IMG, 3 * W), randn(TXT, 3 * W)
        ws = [randn(HEAD_DIM, std=0.05, mean=1.0) for _ in range(4)]
        tabs = [torch.rand(n, HEAD_DIM // 2, generator=g, device=dev) for n in (IMG, IMG, TXT, TXT)]

        def stream(packed, wq, wk, c, s):
            outs = []
            for part, w in ((0, wq), (1, wk)):
                t = packed[:, part * W:(part + 1) * W].unflatten(-1, (HEADS, HEAD_DIM))
                n = (F.rms_norm(t.float(), (HEAD_DIM,), eps=1e-6) * w.float()).to(bf16)
                p = n.float().unflatten(-1, (HEAD_DIM // 2, 2))
                cc, ss = c[:, None, :], s[:, None, :]
                o = torch.stack((p[..., 0] * cc - p[..., 1] * ss, p[..., 1] * cc + p[..., 0] * ss), -1)
                outs.append(o.flatten(-2).to(bf16))
            outs.append(packed[:, 2 * W:].unflatten(-1, (HEADS, HEAD_DIM)))
            return outs

        def run():
            ti = stream(txt, ws[2], ws[3], tabs[2], tabs[3])
            ii = stream(img, ws[0], ws[1], tabs[0], tabs[1])
            return [torch.cat([t, i], 0) for t, i in zip(ti, ii)]
        return run

    def mk_bma():
        x, res = randn(IMG + TXT, H), randn(IMG + TXT, H)
        b, gt = randn(H, std=0.02), randn(H, std=0.5)
        return lambda: (x + b) * gt + res

    def mk_cat_fp8():
        a, m = randn(FLUX_ROWS, FLUX_A), randn(FLUX_ROWS, FLUX_B)
        return lambda: quant(torch.cat([a, m], 1), 20.0)

    pipelines = {"norm_img": (mk_norm, bytes_norm(IMG, H)), "sr_norm": (mk_sr, bytes_sr(IMG, H)),
                 "qkv": (mk_qkv, bytes_qkv(IMG + TXT, HEADS, HEAD_DIM)),
                 "bma": (mk_bma, bytes_bma(IMG + TXT, H)),
                 "cat_fp8": (mk_cat_fp8, bytes_cat_fp8(FLUX_ROWS, FLUX_A + FLUX_B))}
    out = {}
    for name, (mk, nbytes) in pipelines.items():
        try:
            sets = [mk() for _ in range(-(-ROTATION_BYTES // nbytes))]
            for f in sets:
                f()
            ms, _ = time_launches(torch, sets, max(50, 2 * len(sets)))
            out[name] = {"us_per_call": round(1e3 * ms, 3),
                         "gb_s_of_fused_bytes": round(nbytes / (ms * 1e-3) / 1e9, 1)}
            del sets
        except (RuntimeError, TypeError) as e:  # a dtype or op this PyTorch build lacks
            out[name] = {"error": str(e)[:200]}
    torch.cuda.empty_cache()
    return out


def extra_timings(torch, qe, steps):
    """Isolated per-launch timings of the kernels timed beside the step."""
    ex = Workload(torch, qe, seed=0, names=Workload.EXTRA)
    ext = kernel_timings(torch, qe, ex, steps)
    extra = {}
    for name, nbytes, _ in ex.launches:
        iso = ext[name]["iso_ms"]
        extra[name] = {"us_per_call": round(1e3 * iso, 3), "us_passes": pass_range_us(ext[name]),
                       "bytes": nbytes, "gb_s": round(nbytes / (iso * 1e-3) / 1e9, 1),
                       "pct_peak": round(100 * nbytes / (iso * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
                       "rotation_sets": ext[name]["sets"]}
        if nbytes < 32 << 20:  # short launches: also without the Python launch cost
            extra[name]["graph_us_per_call"] = round(graph_us_per_call(torch, qe, name, nbytes), 3)
    return extra


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-sample-div", type=int, default=2,
                    help="the CPU oracle runs on 1/N of each epilogue's rows")
    ap.add_argument("--only", default="", help="comma-separated subset of launches to time")
    ap.add_argument("--print-source-hashes", action="store_true",
                    help="print the source hash of every launch's kernel and exit")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the kernels timed beside the step (FLUX.2 QKV, output selections)")
    ap.add_argument("--extra-only", action="store_true",
                    help="time only the kernels timed beside the step, each in isolation")
    ap.add_argument("--no-split", action="store_true",
                    help="skip the PyTorch split-path timings")
    ap.add_argument("--step-only", action="store_true",
                    help="time the step only, no per-kernel timing (for counter runs)")
    ap.add_argument("--blocks", type=int, default=60,
                    help="also time a Qwen-Image block sequence of this many blocks (0: skip)")
    args = ap.parse_args()
    if args.print_source_hashes:
        print(json.dumps({n: kernel_source_hash(n) for n in KERNEL_SOURCES}))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: these epilogues need no cross-GPU exchange and "
              "each launch runs on one MI355X; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import quant_epilogues_amd as qe

    qe.lib()
    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration(torch)
        return
    if args.extra_only:
        print(json.dumps({"metric": METRIC, "extra_kernels": extra_timings(torch, qe, args.steps)}),
              flush=True)
        return
    names = tuple(args.only.split(",")) if args.only else Workload.ALL
    wl = Workload(torch, qe, seed=0, names=names)
    for _ in range(args.warmup):
        wl.step()
    settle_steps, settle_trace = settle(torch, wl)
    ms, wall = time_steps(torch, wl, args.steps)  # the headline: exactly --steps steps
    value = wl.step_bytes / (ms * 1e-3) / 1e9
    windows = [time_steps(torch, wl, args.steps)[0] for _ in range(SPREAD_WINDOWS)]
    spread = {"windows": SPREAD_WINDOWS, "steps_per_window": args.steps,
              "ms_per_step": [round(w, 4) for w in windows],
              "min_ms": round(min(windows), 4), "max_ms": round(max(windows), 4)}
    if args.step_only:
        print(json.dumps({"metric": METRIC, "value": round(value, 1), "unit": "GB/s",
                          "ms_per_step": round(ms, 4), "steps": args.steps,
                          "settle_steps": settle_steps, "settle_trace_ms": settle_trace,
                          "spread": spread}), flush=True)
        return
    timings = kernel_timings(torch, qe, wl, args.steps)

    kernels = {}
    for name, nbytes, _ in wl.launches:
        t = timings[name]
        iso = t["iso_ms"]
        kernels[name] = {"us_per_call": round(1e3 * iso, 3), "us_passes": pass_range_us(t),
                         "bytes": nbytes, "gb_s": round(nbytes / (iso * 1e-3) / 1e9, 1),
                         "pct_peak": round(100 * nbytes / (iso * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
                         "rotation_sets": t["sets"]}
        if nbytes < 32 << 20:  # short launches: also without the Python launch cost
            kernels[name]["graph_us_per_call"] = round(graph_us_per_call(torch, qe, name, nbytes), 3)
    # The block sequence is timed right after the step's own launches, at the
    # same steady state as the headline; the kernels beside the step, the
    # short-row norms and the split path (about 20 s more of load) come after.
    blocks = block_sequence(torch, qe, args.blocks, reps=5) if args.blocks else None
    extra = {} if args.only or args.no_extra else extra_timings(torch, qe, args.steps)
    norm_rows = {} if args.only or args.no_extra else norm_rows_timings(torch, qe, args.steps)
    split = {}
    if not args.only and not args.no_split:
        log("timing the PyTorch split path ...")
        split = split_path_timings(torch, args.steps)
        for name, rec in split.items():
            fused = kernels.get(name) or extra.get(name)
            if "us_per_call" in rec and fused:
                rec["fused_us_per_call"] = fused["us_per_call"]
                rec["fused_speedup"] = round(rec["us_per_call"] / fused["us_per_call"], 2)
    dom = max(kernels, key=lambda n: kernels[n]["us_per_call"])
    achieved = kernels[dom]["gb_s"]
    traffic = profiled_traffic(dom)
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded randn, resident in HBM)",
        "config": {"workload": "Qwen-Image block epilogues (hidden 3072, 512 text + 4096 image "
                               "tokens, 24x128 heads) + FLUX.2 single-block token-cat FP8/FP4 "
                               "(4608 x 6144+18432)",
                   "launches_per_step": len(wl.launches), "step_bytes": wl.step_bytes,
                   "io": "bf16 in; bf16 + E4M3 / E2M1 out", "parallelism": "1 GPU"},
        "pct_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "wall_ms_per_step": round(1e3 * wall, 4),
        "settle_steps": settle_steps, "settle_trace_ms": settle_trace, "spread": spread,
        "kernels": kernels,
        "extra_kernels": extra,
        "norm_rows": norm_rows,
        "split_path": split,
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "algorithmic_bytes": kernels[dom]["bytes"]},
    }
    if blocks:
        out["block_sequence"] = blocks
    if not args.no_cpu:
        log("timing the CPU oracle on a row sample ...")
        out["cpu_baseline"] = cpu_baseline(args.cpu_sample_div)
        out["cpu_baseline_all_cores"] = cpu_baseline(args.cpu_sample_div, cpu_threads())
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

"""bench.py's compulsory-byte accounting and its command-line contract (CPU).

The byte counts are what every GB/s and roofline figure divides by, so they
are pinned here to the counts derived independently from the shapes (each
input read once, each output written once, row-broadcast vectors once):
  LN + FP8, 4096 x 3072: x 2 B + y 2 B + q 1 B per element, scale/shift 2 x 6 KiB,
    the fp32 input scale 4 B;
  the same at 127 rows (the latency case);
  bias + gated residual + LN + FP8, 4096 x 3072: x, residual, r, y 2 B each + q 1 B,
    bias/gate/scale/shift 4 x 6 KiB, 4 B scale;
  QKV epilogue, 4608 tokens x 24 heads x 128: Q/K/V read and written (12 B per
    element of one part) + 4 RMSNorm weights + fp32 cos/sin [4608, 64] each;
  bias_mul_add, 4608 x 3072: x, residual, y 2 B each + bias/gate;
  token-cat FP8, 4608 x 24576: 2 B in, 1 B out; FP4: 2 B in, 0.5 B codes,
    one scale byte per 16 elements over rows padded to 128.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_compulsory_bytes_match_the_shapes():
    H = 3072
    vec = 2 * H
    assert bench.bytes_norm(4096, H) == 5 * 4096 * H + 2 * vec + 4
    assert bench.bytes_norm(127, H) == 5 * 127 * H + 2 * vec + 4
    assert bench.bytes_norm(4608, 6144, y=False) == 3 * 4608 * 6144 + 2 * 2 * 6144 + 4
    assert bench.bytes_sr(4096, H) == 9 * 4096 * H + 4 * vec + 4
    assert bench.bytes_sr(4096, H, q=False) == 8 * 4096 * H + 4 * vec
    tokens, heads, d = 4608, 24, 128
    assert bench.bytes_qkv(tokens, heads, d) == (12 * tokens * heads * d + 4 * 2 * d
                                                 + 2 * 4 * tokens * (d // 2))
    assert bench.bytes_bma(4608, H) == 6 * 4608 * H + 2 * vec
    C = 6144 + 18432
    assert bench.bytes_cat_fp8(4608, C) == 3 * 4608 * C + 4
    assert bench.bytes_cat_fp4(4608, C) == 2 * 4608 * C + 4608 * C // 2 + 4608 * (C // 16) + 4
    assert bench.bytes_cat_fp4(17, 64) == 2 * 17 * 64 + 17 * 32 + 128 * 4 + 4  # pad rows to 128


def test_compulsory_bytes_at_the_stated_megabytes():
    """The rounded figures the measurement plan states for each configuration."""
    mb = lambda b: round(b / 1e6, 2)
    assert mb(bench.bytes_norm(127, 3072)) == 1.96
    assert mb(bench.bytes_norm(4096, 3072)) == 62.93
    assert mb(bench.bytes_sr(4096, 3072)) == 113.27  # 113 270 788 B (the plan prints 113.28)
    assert mb(bench.bytes_qkv(4608, 24, 128)) == 172.23
    assert mb(bench.bytes_bma(4608, 3072)) == 84.95
    assert mb(bench.bytes_cat_fp8(4608, 24576)) == 339.74
    assert mb(bench.bytes_cat_fp4(4608, 24576)) == 290.19


def test_more_than_one_gpu_is_refused_with_a_message():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr


def test_kernel_sources_cover_every_launch():
    names = set(bench.Workload.ALL) | set(bench.Workload.EXTRA)
    assert names <= set(bench.KERNEL_SOURCES)
    for n in names:
        assert len(bench.kernel_source_hash(n)) == 16

"""The C ABI without a GPU: the library loads, exports every function the
header declares, and refuses bad arguments on the host before any HIP call.

Only refusals and rows == 0 calls are made here (both return before touching
HIP), with fake but aligned device addresses. The module is skipped where a GPU
is visible so that no fake address can ever reach a kernel.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _gpu_visible() -> bool:
    import torch

    return torch.cuda.device_count() > 0


pytestmark = pytest.mark.skipif(_gpu_visible(), reason="host-only refusal tests use fake device addresses")

FAKE = 0x7F0000000000  # 16-byte aligned, never dereferenced
FAKE2 = FAKE + 0x100000


@pytest.fixture(scope="module")
def native():
    from quant_epilogues_amd import _native

    if not os.path.exists(_native.LIB_PATH):
        from quant_epilogues_amd import _build

        _build.build()
    _native.lib()
    return _native


def test_exports_every_declared_symbol(native):
    declared = native.header_symbols()
    assert set(declared) == {
        "dit_abi_version", "dit_status_string", "dit_last_error", "dit_norm_modulate_fp8",
        "dit_norm_modulate_fp8_dual", "dit_scale_residual_norm_modulate_fp8", "dit_norm_modulate_fp4",
        "dit_scale_residual_norm_modulate_fp4", "dit_qkv_epilogue", "dit_bias_mul_add",
        "dit_token_cat_quant",
    }
    raw = ctypes.CDLL(native.LIB_PATH)
    for name in declared:
        assert hasattr(raw, name), name


def test_version_and_status_strings(native):
    L = native.lib()
    with open(os.path.join(ROOT, "include", "dit_epilogues.h")) as f:
        ver = int(re.search(r"#define DIT_ABI_VERSION (\d+)", f.read()).group(1))
    assert L.dit_abi_version() == ver
    names = [native.status_string(s) for s in range(6)]
    assert names == ["DIT_OK", "DIT_ERR_NULL", "DIT_ERR_SHAPE", "DIT_ERR_ALIGN",
                     "DIT_ERR_UNSUPPORTED", "DIT_ERR_HIP"]
    assert native.status_string(99) == "DIT_ERR_UNKNOWN"


def _nm(L, **kw):
    a = dict(y=FAKE, q=FAKE, x=FAKE, scale=FAKE, shift=FAKE, s=FAKE, rows=4, hidden=3072, eps=1e-6)
    a.update(kw)
    return L.dit_norm_modulate_fp8(a["y"], a["q"], a["x"], a["scale"], a["shift"], a["s"],
                                   a["rows"], a["hidden"], a["eps"], None)


def test_norm_modulate_refusals(native):
    L = native.lib()
    assert _nm(L, x=None) == native.DIT_ERR_NULL
    assert "NULL" in native.last_error()
    assert _nm(L, rows=-1) == native.DIT_ERR_SHAPE
    assert _nm(L, hidden=0) == native.DIT_ERR_SHAPE
    assert _nm(L, hidden=3076) == native.DIT_ERR_UNSUPPORTED
    assert _nm(L, hidden=8200) == native.DIT_ERR_UNSUPPORTED
    assert _nm(L, x=FAKE + 2) == native.DIT_ERR_ALIGN
    assert _nm(L, q=FAKE + 8) == native.DIT_ERR_ALIGN
    assert _nm(L, s=FAKE + 2) == native.DIT_ERR_ALIGN
    assert _nm(L, rows=0) == native.DIT_OK  # no-op, no HIP call
    assert native.last_error() == ""
    # Either output may be left out, not both; q needs the scale.
    assert _nm(L, y=None, q=None) == native.DIT_ERR_NULL
    assert _nm(L, s=None) == native.DIT_ERR_NULL
    assert _nm(L, y=None, rows=0) == native.DIT_OK
    assert _nm(L, q=None, s=None, rows=0) == native.DIT_OK


def _dual(L, **kw):
    a = dict(iy=FAKE, iq=FAKE, ix=FAKE, isc=FAKE, ish=FAKE, iss=FAKE, irows=8,
             ty=FAKE, tq=FAKE, tx=FAKE, tsc=FAKE, tsh=FAKE, tss=FAKE, trows=2, hidden=3072)
    a.update(kw)
    return L.dit_norm_modulate_fp8_dual(a["iy"], a["iq"], a["ix"], a["isc"], a["ish"], a["iss"],
                                        a["irows"], 1e-6, a["ty"], a["tq"], a["tx"], a["tsc"],
                                        a["tsh"], a["tss"], a["trows"], 1e-5, a["hidden"], None)


def test_norm_modulate_dual_refusals(native):
    L = native.lib()
    assert _dual(L, ix=None) == native.DIT_ERR_NULL
    assert "img" in native.last_error()
    assert _dual(L, tsc=None) == native.DIT_ERR_NULL
    assert "txt" in native.last_error()
    assert _dual(L, ty=None, tq=None) == native.DIT_ERR_NULL
    assert _dual(L, iss=None) == native.DIT_ERR_NULL  # q needs its scale
    assert _dual(L, irows=-1) == native.DIT_ERR_SHAPE
    assert _dual(L, hidden=3076) == native.DIT_ERR_UNSUPPORTED
    assert _dual(L, tx=FAKE + 2) == native.DIT_ERR_ALIGN
    assert _dual(L, irows=0, trows=0) == native.DIT_OK
    # A stream with no rows needs no pointers; the other is still checked.
    assert _dual(L, irows=0, trows=0, ix=None, tx=None) == native.DIT_OK
    assert _dual(L, irows=0, ix=None, iy=None, iq=None, tx=FAKE + 8) == native.DIT_ERR_ALIGN
    assert _dual(L, irows=1 << 30) == native.DIT_ERR_UNSUPPORTED
    assert _dual(L, irows=1 << 62, trows=1 << 62) == native.DIT_ERR_UNSUPPORTED  # no overflow


def test_scale_residual_refusals(native):
    L = native.lib()
    f = L.dit_scale_residual_norm_modulate_fp8
    args = [FAKE] * 10 + [4, 3072, 1e-6, None]
    bad = list(args)
    bad[0] = None
    assert f(*bad) == native.DIT_ERR_NULL
    bad = list(args)
    bad[4] = FAKE + 4  # misaligned bias
    assert f(*bad) == native.DIT_ERR_ALIGN
    bad = list(args)
    bad[4] = None  # bias is optional
    bad[10] = 0
    assert f(*bad) == native.DIT_OK
    bad = list(args)
    bad[11] = 12
    assert f(*bad) == native.DIT_ERR_UNSUPPORTED
    bad = list(args)
    bad[1] = bad[2] = None  # neither y nor q
    assert f(*bad) == native.DIT_ERR_NULL
    bad = list(args)
    bad[2] = bad[9] = None  # bf16 only, no scale needed
    bad[10] = 0
    assert f(*bad) == native.DIT_OK


def _qkv(L, **kw):
    a = dict(heads=24, head_dim=128, img_rows=8, txt_rows=2, img_stride=9216, txt_stride=9216,
             img_q=FAKE, txt_q=FAKE, jq=FAKE, img_cos=FAKE, rope_stride=64)
    a.update(kw)
    return L.dit_qkv_epilogue(a["jq"], FAKE, FAKE, a["img_q"], FAKE, FAKE, a["img_rows"],
                              a["img_stride"], a["txt_q"], FAKE, FAKE, a["txt_rows"],
                              a["txt_stride"], FAKE, FAKE, FAKE, FAKE, a["img_cos"], FAKE, FAKE,
                              FAKE, a["rope_stride"], a["heads"], a["head_dim"], 1e-6, 1e-6, None)


def test_qkv_refusals(native):
    L = native.lib()
    assert _qkv(L, head_dim=64) == native.DIT_ERR_UNSUPPORTED  # only 128
    assert _qkv(L, heads=0) == native.DIT_ERR_UNSUPPORTED
    assert _qkv(L, heads=65) == native.DIT_ERR_UNSUPPORTED
    assert _qkv(L, img_stride=3000) == native.DIT_ERR_SHAPE
    assert _qkv(L, txt_stride=9220) == native.DIT_ERR_SHAPE
    assert _qkv(L, img_rows=-1) == native.DIT_ERR_SHAPE
    assert _qkv(L, jq=None) == native.DIT_ERR_NULL
    assert _qkv(L, img_q=None) == native.DIT_ERR_NULL
    assert _qkv(L, img_cos=FAKE + 4) == native.DIT_ERR_ALIGN
    assert _qkv(L, rope_stride=32) == native.DIT_ERR_SHAPE  # shorter than head_dim / 2
    assert _qkv(L, rope_stride=66) == native.DIT_ERR_SHAPE  # rows not 16-byte aligned
    assert _qkv(L, rope_stride=128, img_rows=0, txt_rows=0) == native.DIT_OK
    # A stream with no rows needs no pointers.
    assert _qkv(L, img_rows=0, txt_rows=0, img_q=None, txt_q=None) == native.DIT_OK


def test_bias_mul_add_refusals(native):
    L = native.lib()
    f = L.dit_bias_mul_add
    assert f(None, FAKE, FAKE, FAKE, FAKE, 4, 3072, None) == native.DIT_ERR_NULL
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 3071, None) == native.DIT_ERR_UNSUPPORTED
    assert f(FAKE, FAKE, FAKE + 2, FAKE, FAKE, 4, 3072, None) == native.DIT_ERR_ALIGN
    assert f(FAKE, FAKE, None, FAKE, FAKE, 0, 3072, None) == native.DIT_OK


def test_token_cat_refusals(native):
    L = native.lib()
    f = L.dit_token_cat_quant
    fp8, fp4 = native.DIT_QUANT_FP8_E4M3, native.DIT_QUANT_FP4_E2M1
    assert f(7, FAKE, None, FAKE, 6144, FAKE2, 18432, 4, FAKE, None) == native.DIT_ERR_UNSUPPORTED
    assert f(fp8, FAKE, None, FAKE, 6140, FAKE2, 18432, 4, FAKE, None) == native.DIT_ERR_SHAPE
    assert f(fp8, FAKE, None, FAKE, 0, FAKE2, 16, 4, FAKE, None) == native.DIT_ERR_SHAPE
    assert f(fp4, FAKE, None, FAKE, 6144, FAKE2, 18432, 4, FAKE, None) == native.DIT_ERR_NULL
    assert f(fp8, FAKE, None, FAKE, 6144, None, 18432, 4, FAKE, None) == native.DIT_ERR_NULL
    assert f(fp8, FAKE + 8, None, FAKE, 6144, FAKE2, 18432, 4, FAKE, None) == native.DIT_ERR_ALIGN
    assert f(fp4, FAKE, FAKE, FAKE, 6144, None, 0, 0, FAKE, None) == native.DIT_OK
    huge = (1 << 62) + 16  # a multiple of 16 whose sum with itself overflows int64
    assert f(fp8, FAKE, None, FAKE, huge, FAKE2, huge, 4, FAKE, None) == native.DIT_ERR_UNSUPPORTED


def test_python_binding_has_no_cpu_path(native):
    import torch

    import quant_epilogues_amd as qe

    x = torch.zeros(4, 3072, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        qe.norm_modulate_fp8(x, x[0], x[0], torch.ones(1), 1e-6)


def test_refuses_launches_beyond_the_grid_limit(native):
    # Each launch covers at most 2^32 lanes; larger sizes are refused on the
    # host with DIT_ERR_UNSUPPORTED instead of failing inside HIP.
    L = native.lib()
    big = 1 << 30
    assert _nm(L, rows=big) == native.DIT_ERR_UNSUPPORTED
    assert "grid limit" in native.last_error()
    f = L.dit_scale_residual_norm_modulate_fp8
    assert f(*([FAKE] * 10 + [big, 3072, 1e-6, None])) == native.DIT_ERR_UNSUPPORTED
    assert _qkv(L, img_rows=1 << 27) == native.DIT_ERR_UNSUPPORTED
    assert L.dit_bias_mul_add(FAKE, FAKE, None, FAKE, FAKE, big, 3072, None) == native.DIT_ERR_UNSUPPORTED
    assert "grid limit" in native.last_error()
    # Token concatenation splits rows over several launches; its limits are
    # the row count (2^31 - 128) and the row width (2^28).
    cat = L.dit_token_cat_quant
    assert cat(native.DIT_QUANT_FP8_E4M3, FAKE, None, FAKE, 6144, FAKE2, 18432, 1 << 31, FAKE,
               None) == native.DIT_ERR_UNSUPPORTED
    assert cat(native.DIT_QUANT_FP4_E2M1, FAKE, FAKE, FAKE, 1 << 28, FAKE2, 16, 4, FAKE,
               None) == native.DIT_ERR_UNSUPPORTED


def test_norm_fp4_refusals(native):
    L = native.lib()
    f = L.dit_norm_modulate_fp4
    row_major, tiled = native.DIT_FP4_SCALES_ROW_MAJOR, native.DIT_FP4_SCALES_128X4
    args = [FAKE, FAKE, FAKE, row_major, FAKE, FAKE, FAKE, FAKE, 4, 3072, 1e-6, None]
    bad = list(args)
    bad[1] = None  # packed
    assert f(*bad) == native.DIT_ERR_NULL
    bad = list(args)
    bad[9] = 3080  # a multiple of 8, not of 16
    assert f(*bad) == native.DIT_ERR_UNSUPPORTED
    bad = list(args)
    bad[3], bad[9] = tiled, 3088  # 193 groups: not whole 128x4 tiles
    assert f(*bad) == native.DIT_ERR_UNSUPPORTED
    bad = list(args)
    bad[3] = 7  # no such layout
    assert f(*bad) == native.DIT_ERR_UNSUPPORTED
    bad = list(args)
    bad[1] = FAKE + 8
    assert f(*bad) == native.DIT_ERR_ALIGN
    bad = list(args)
    bad[2] = FAKE + 3  # scales may have any alignment
    bad[8] = 0
    assert f(*bad) == native.DIT_OK
    g = L.dit_scale_residual_norm_modulate_fp4
    args = [FAKE] * 4 + [row_major] + [FAKE] * 7 + [4, 3072, 1e-6, None]
    bad = list(args)
    bad[7] = None  # gate
    assert g(*bad) == native.DIT_ERR_NULL
    bad = list(args)
    bad[1] = bad[6] = None  # no y, no bias
    bad[12] = 0
    assert g(*bad) == native.DIT_OK
    assert g(*(args[:12] + [1 << 30, 3072, 1e-6, None])) == native.DIT_ERR_UNSUPPORTED


def test_token_cat_tiled_scales_need_whole_tiles(native):
    L = native.lib()
    f = L.dit_token_cat_quant
    tiled = native.DIT_QUANT_FP4_E2M1_128X4
    assert f(tiled, FAKE, FAKE, FAKE, 6144, FAKE2, 16, 4, FAKE, None) == native.DIT_ERR_UNSUPPORTED
    assert f(tiled, FAKE, FAKE, FAKE, 6144, FAKE2, 18432, 0, FAKE, None) == native.DIT_OK
    assert f(tiled, FAKE, FAKE + 8, FAKE, 6144, FAKE2, 18432, 4, FAKE, None) == native.DIT_ERR_ALIGN
    assert f(3, FAKE, FAKE, FAKE, 6144, FAKE2, 18432, 4, FAKE, None) == native.DIT_ERR_UNSUPPORTED


_NO_DEVICE_SCRIPT = r"""
import ctypes, json, sys
sys.path.insert(0, sys.argv[1])
count = ctypes.c_int(0)
rc = ctypes.CDLL("libamdhip64.so").hipGetDeviceCount(ctypes.byref(count))
if rc == 0 and count.value > 0:  # a device is visible: never pass it fake addresses
    print(json.dumps({"device_visible": True}))
    sys.exit(0)
from quant_epilogues_amd import _native as nat
L = nat.lib()
F, F2 = 0x7F0000000000, 0x7F0000100000
calls = {
    "dit_norm_modulate_fp8": lambda: L.dit_norm_modulate_fp8(F, F, F, F, F, F, 4, 3072, 1e-6, None),
    "dit_norm_modulate_fp8_dual": lambda: L.dit_norm_modulate_fp8_dual(
        F, F, F, F, F, F, 8, 1e-6, F, F, F, F, F, F, 2, 1e-6, 3072, None),
    "dit_scale_residual_norm_modulate_fp8": lambda: L.dit_scale_residual_norm_modulate_fp8(
        *([F] * 10 + [4, 3072, 1e-6, None])),
    "dit_norm_modulate_fp4": lambda: L.dit_norm_modulate_fp4(
        F, F, F, nat.DIT_FP4_SCALES_ROW_MAJOR, F, F, F, F, 4, 3072, 1e-6, None),
    "dit_scale_residual_norm_modulate_fp4": lambda: L.dit_scale_residual_norm_modulate_fp4(
        *([F] * 4 + [nat.DIT_FP4_SCALES_128X4] + [F] * 7 + [4, 3072, 1e-6, None])),
    "dit_qkv_epilogue": lambda: L.dit_qkv_epilogue(
        F, F, F, F, F, F, 8, 9216, F, F, F, 2, 9216, F, F, F, F, F, F, F, F, 64, 24, 128,
        1e-6, 1e-6, None),
    "dit_bias_mul_add": lambda: L.dit_bias_mul_add(F, F, F, F, F, 4, 3072, None),
    "dit_token_cat_quant": lambda: L.dit_token_cat_quant(
        nat.DIT_QUANT_FP4_E2M1, F, F2, F, 6144, F2, 18432, 4, F, None),
}
out = {}
for name, call in calls.items():
    status = call()
    out[name] = [status, nat.last_error()]
print(json.dumps({"device_visible": False, "calls": out}))
"""


def test_launch_failure_reports_dit_err_hip():
    """With no GPU visible to HIP, every compute entry point passes its host
    checks and then returns DIT_ERR_HIP with the runtime's reason: a failed
    launch is reported, never silent. Runs in a child process whose HIP sees
    no device; it asks HIP for the device count first and makes no call at all
    if a device is visible."""
    import json
    import subprocess
    import sys

    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1", ROCR_VISIBLE_DEVICES="-1")
    p = subprocess.run([sys.executable, "-c", _NO_DEVICE_SCRIPT, ROOT], env=env,
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 0, p.stderr[-2000:]
    res = json.loads(p.stdout.strip().splitlines()[-1])
    if res["device_visible"]:
        pytest.skip("HIP still sees a device in the child process")
    assert set(res["calls"]) == {n for n in _native_symbols() if n not in (
        "dit_abi_version", "dit_status_string", "dit_last_error")}
    for name, (status, msg) in res["calls"].items():
        assert status == 5, (name, status, msg)  # DIT_ERR_HIP
        assert name in msg and "launch failed" in msg, (name, msg)


def _native_symbols():
    from quant_epilogues_amd import _native

    return _native.header_symbols()

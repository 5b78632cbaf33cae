"""The library's conversion helpers (quant_epilogues_amd/csrc/dit_device.h)
against the CPU oracle's encoders, on dense sweeps of inputs.

The helpers run in a test-only library (tests/native/conversions.hip) that
includes the same header the kernels use. div6_bf16 is also compiled for the
host and checked there, exhaustively, without a GPU.

Sweep: every fp32 value whose upper 16 bits are any finite pattern and whose
lower 16 bits lie within 2 ulps of 0x0000 or 0x8000, plus 2^22 random finite
fp32 values. That holds every bf16 value, every bf16 rounding midpoint with
its neighbours, and every E4M3 and E2M1 rounding boundary with its
neighbours: those boundaries have at most 5 significant bits, so their lower
16 bits are zero.
"""
import ctypes
import os

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def _lib():
    from native import build as nb

    if not os.path.exists(nb.LIB_PATH):
        nb.build()
    L = ctypes.CDLL(nb.LIB_PATH)
    L.dit_cvt_sweep.restype = ctypes.c_int
    L.dit_cvt_sweep.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                ctypes.c_void_p]
    L.dit_div6_host.restype = None
    L.dit_div6_host.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64]
    return L


def _nonneg_bf16_values() -> np.ndarray:
    """Every non-negative finite bf16 value (subnormals included) and +inf, as fp32."""
    bits = np.arange(0, 0x7F81, dtype=np.uint32)  # 0x7F80 = +inf
    return (bits << 16).view(np.float32)


def _sweep() -> np.ndarray:
    hi = np.arange(65536, dtype=np.uint32)
    hi = hi[(hi & 0x7F80) != 0x7F80]  # finite upper halves
    lows = np.array([0x0000, 0x0001, 0x0002, 0xFFFE, 0xFFFF,
                     0x7FFE, 0x7FFF, 0x8000, 0x8001, 0x8002], np.uint32)
    dense = ((hi[:, None] << 16) | lows[None, :]).ravel()
    rnd = np.random.default_rng(2024).integers(0, 2**32, 1 << 22, dtype=np.uint64).astype(np.uint32)
    rnd = rnd[(rnd & 0x7F800000) != 0x7F800000]
    v = np.concatenate([dense, rnd]).view(np.float32)
    return v[: v.size // 8 * 8]


def test_div6_bf16_on_the_host_is_the_ieee_quotient():
    """div6_bf16 (a product with RN(1/6) and one FMA correction) equals IEEE
    fp32 a / 6 for every non-negative finite bf16 value, +inf included."""
    L = _lib()
    a = _nonneg_bf16_values()
    out = np.empty_like(a)
    L.dit_div6_host(a.ctypes.data, out.ctypes.data, a.size)
    want = a / np.float32(6.0)  # numpy binary32 division: IEEE, round to nearest even
    assert want.dtype == np.float32
    assert np.array_equal(out.view(np.uint32), want.view(np.uint32))


@pytest.mark.gpu
class TestOnTheGpu:
    @pytest.fixture(scope="class")
    def dev(self):
        import torch

        if not torch.cuda.is_available():
            pytest.skip("no GPU visible")
        return torch

    def _run(self, torch, kind, v, out_elems, out_dtype):
        L = _lib()
        vin = torch.from_numpy(np.ascontiguousarray(v)).cuda()
        out = torch.empty(out_elems, dtype=out_dtype, device="cuda")
        print(f"case: conversion sweep kind {kind}, {v.size} values", flush=True)
        rc = L.dit_cvt_sweep(kind, vin.data_ptr(), out.data_ptr(), v.size,
                             torch.cuda.current_stream().cuda_stream)
        assert rc == 0, rc
        torch.cuda.synchronize()
        return out.cpu().numpy()

    def test_e4m3_clamp_and_pack(self, dev, oracle_mod):
        v = _sweep()
        got = self._run(dev, 0, v, v.size // 4, dev.int32).view(np.uint8)
        want = oracle_mod.e4m3_encode(v)  # saturates at +-448 like the clamp
        assert np.array_equal(got, want)

    def test_e2m1_pack(self, dev, oracle_mod):
        v = _sweep()
        got = self._run(dev, 1, v, v.size // 8, dev.int32).view(np.uint8)
        nib = np.stack([got & 0xF, got >> 4], axis=-1).ravel()
        want = oracle_mod.e2m1_encode(v)
        assert np.array_equal(nib, want)

    def test_bf16_pack_and_round(self, dev, oracle_mod):
        v = _sweep()
        got = self._run(dev, 2, v, v.size // 2, dev.int32).view(np.uint16)
        want = oracle_mod.bf16_from_f32(v)
        assert np.array_equal(got, want)
        got_r = self._run(dev, 3, v, v.size, dev.float32)
        assert np.array_equal(got_r.view(np.uint32), want.astype(np.uint32) << 16)

    def test_div6_bf16(self, dev):
        a = _nonneg_bf16_values()
        got = self._run(dev, 4, a, a.size, dev.float32)
        assert np.array_equal(got.view(np.uint32), (a / np.float32(6.0)).view(np.uint32))

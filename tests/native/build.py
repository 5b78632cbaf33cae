"""Build the test-only conversion-sweep library (tests/native/libdit_cvtcheck.so)
with the product library's compiler flags, against its device helpers."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdit_cvtcheck.so")


def build(verbose: bool = False) -> str:
    from quant_epilogues_amd import _build as B

    cmd = [B._hipcc(), *B.HIPFLAGS, "-shared", os.path.join(HERE, "conversions.hip"), "-o",
           LIB_PATH + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed on conversions.hip:\n" + res.stderr[-3000:])
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH

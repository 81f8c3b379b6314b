"""Exhaustive CPU check of the rounding identity behind the requantisation
kernel's code computation (tests/exhaustive/requant_rounding.c): over every
finite binary16 scale (zero, subnormal and normal, plus infinity) and every
finite binary16 or bfloat16 weight, the kernel's W * (1/s) snapped to 2^-14
and rounded to nearest even gives the same int4 code as the definition
clamp(round_half_even(fl32(W / s)), -7, 7).  This is what lets the kernel
resolve exact ties (W / s a half-integer, frequent for binary16 inputs)
without a division."""
import ctypes
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "exhaustive", "requant_rounding.c")
LIB = os.path.join(HERE, "exhaustive", "librequant_rounding.so")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
                        "-shared", "-fPIC", SRC, "-o", LIB, "-lm"], check=True)
    L = ctypes.CDLL(LIB)
    L.count_mismatches.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   ctypes.POINTER(ctypes.c_uint32), ctypes.POINTER(ctypes.c_uint32)]
    L.count_mismatches.restype = ctypes.c_longlong
    return L


def _run(lib, dtype, lo, hi, snap=1):
    fw, fs = ctypes.c_uint32(0xFFFFFFFF), ctypes.c_uint32(0xFFFFFFFF)
    bad = lib.count_mismatches(dtype, lo, hi, snap, ctypes.byref(fw), ctypes.byref(fs))
    return bad, hex(fw.value), hex(fs.value)


def test_without_the_snap_ties_go_wrong(lib):
    """Negative control: rounding W * (1/s) directly (no snap) mis-resolves
    exact ties for some scales, so the comparison can fail."""
    bad, w, s = _run(lib, 0, 0x3000, 0x3400, snap=0)
    assert bad > 0


@pytest.mark.parametrize("dtype", [0, 1], ids=["binary16 weights", "bfloat16 weights"])
def test_every_weight_scale_pair(lib, dtype):
    # every non-negative binary16 scale: +0, subnormals, normals, +inf
    bad, w, s = _run(lib, dtype, 0x0000, 0x7C01)
    assert bad == 0, f"{bad} mismatches, first weight bits {w}, scale bits {s}"

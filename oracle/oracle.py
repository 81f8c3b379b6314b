"""ctypes wrapper around the C oracle (liboracle.so).

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
CPU-baseline leg of the benchmark, never by the GPU library or its binding.
It holds no arithmetic of its own beyond allocating numpy outputs; every
number comes from oracle.c, which follows the definition step by step (see
the header of oracle.c for the passages each step follows).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

OK, EINVAL, EWEIGHT, ENONFINITE = 0, -1, -2, -3

GCC_FLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
             "-shared", "-fPIC"]


def build(verbose: bool = False) -> str:
    """Compile oracle.c into liboracle.so next to it (host gcc)."""
    cmd = ["gcc", *GCC_FLAGS, _SRC, "-o", _LIB_PATH, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return _LIB_PATH


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i32 = ctypes.c_int
        L.oracle_half_to_double.argtypes = [ctypes.c_uint16]
        L.oracle_half_to_double.restype = ctypes.c_double
        L.oracle_unpack.argtypes = [P, i32, i32, P, P]
        L.oracle_unpack.restype = i32
        L.oracle_count_bad_nibbles.argtypes = [P, i32, i32]
        L.oracle_count_bad_nibbles.restype = ctypes.c_int64
        L.oracle_logit_one.argtypes = [P, P, P, i32]
        L.oracle_logit_one.restype = ctypes.c_float
        L.oracle_logits.argtypes = [P, P, P, i32, i32, i32, P, i32]
        L.oracle_logits.restype = i32
        L.oracle_argmax_rows.argtypes = [P, i32, i32, P, P, P, P]
        L.oracle_argmax_rows.restype = i32
        L.oracle_accept.argtypes = [P, P, i32, i32, P]
        L.oracle_accept.restype = i32
        L.oracle_verify.argtypes = [P, P, P, P, i32, i32, i32, i32, P, P, P, P, P, P, i32]
        L.oracle_verify.restype = i32
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


class OracleError(RuntimeError):
    def __init__(self, status):
        names = {EINVAL: "invalid arguments", EWEIGHT: "weight nibble 0x8 (illegal -8)",
                 ENONFINITE: "non-finite hidden or scale value"}
        super().__init__(f"oracle status {status}: {names.get(status, 'unknown')}")
        self.status = status


def half_to_double(bits: int) -> float:
    return lib().oracle_half_to_double(int(bits))


def unpack(packed: np.ndarray, V: int, H: int) -> np.ndarray:
    packed = _c(packed, np.uint8)
    q = np.empty((V, H), np.int8)
    nbad = ctypes.c_int64(0)
    st = lib().oracle_unpack(_p(packed), V, H, _p(q), ctypes.byref(nbad))
    if st not in (OK, EWEIGHT):
        raise OracleError(st)
    return q, int(nbad.value)


def count_bad_nibbles(packed: np.ndarray, V: int, H: int) -> int:
    packed = _c(packed, np.uint8)
    return int(lib().oracle_count_bad_nibbles(_p(packed), V, H))


def logit_one(hidden_row_bits, packed_row, scales_bits, H: int) -> float:
    x = _c(hidden_row_bits, np.uint16)
    w = _c(packed_row, np.uint8)
    s = _c(scales_bits, np.uint16)
    return float(lib().oracle_logit_one(_p(x), _p(w), _p(s), H))


def logits(hidden_bits, packed, scales_bits, M: int, V: int, H: int, n_threads: int = 0):
    x = _c(hidden_bits, np.uint16)
    w = _c(packed, np.uint8)
    s = _c(scales_bits, np.uint16)
    out = np.empty((M, V), np.float32)
    st = lib().oracle_logits(_p(x), _p(w), _p(s), M, V, H, _p(out), int(n_threads))
    if st != OK:
        raise OracleError(st)
    return out


def argmax_rows(lg: np.ndarray):
    lg = _c(lg, np.float32)
    M, V = lg.shape
    idx = np.empty(M, np.int32)
    mx = np.empty(M, np.float32)
    gap = np.empty(M, np.float32)
    amax = np.empty(M, np.float32)
    st = lib().oracle_argmax_rows(_p(lg), M, V, _p(idx), _p(mx), _p(gap), _p(amax))
    if st != OK:
        raise OracleError(st)
    return idx, mx, gap, amax


def accept(argmax_ids, draft_ids, R: int, T: int) -> np.ndarray:
    a = _c(argmax_ids, np.int32)
    d = None if T == 1 else _c(draft_ids, np.int32)
    n = np.empty(R, np.int32)
    st = lib().oracle_accept(_p(a), _p(d), R, T, _p(n))
    if st != OK:
        raise OracleError(st)
    return n


def verify(hidden_bits, packed, scales_bits, draft_ids, R: int, T: int, V: int, H: int,
           want_logits: bool = False, n_threads: int = 0) -> dict:
    """Full verify step on the host.  Returns a dict with logits_max,
    argmax_ids, n_accepted, gap, amax (and logits when asked)."""
    M = R * T
    x = _c(hidden_bits, np.uint16)
    w = _c(packed, np.uint8)
    s = _c(scales_bits, np.uint16)
    d = None if T == 1 else _c(draft_ids, np.int32)
    lg = np.empty((M, V), np.float32) if want_logits else None
    mx = np.empty(M, np.float32)
    idx = np.empty(M, np.int32)
    n = np.empty(R, np.int32)
    gap = np.empty(M, np.float32)
    amax = np.empty(M, np.float32)
    st = lib().oracle_verify(_p(x), _p(w), _p(s), _p(d), R, T, V, H, _p(lg), _p(mx),
                             _p(idx), _p(n), _p(gap), _p(amax), int(n_threads))
    if st != OK:
        raise OracleError(st)
    out = dict(logits_max=mx, argmax_ids=idx, n_accepted=n, gap=gap, amax=amax)
    if want_logits:
        out["logits"] = lg
    return out

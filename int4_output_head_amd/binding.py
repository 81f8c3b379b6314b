"""Thin Python binding of libint4vh.so (the C ABI declared in include/int4vh.h).

Argument marshalling only: every step of the verify path runs in the HIP
kernels of the library.  torch tensors supply device memory and the current
stream; outputs are allocated with torch on the input's device.  If the
library has not been built the first call raises; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libint4vh.so")

OK, EINVAL, EALIGN, EWORKSPACE, EHIP, EUNSUPPORTED = 0, -1, -2, -3, -4, -5

_lib = None
_lock = threading.Lock()


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load (once) and return the library; raise if it is missing."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with "
                               "`python -c 'import __graft_entry__ as g; g.build()'`")
        L = ctypes.CDLL(path)
        P, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        L.verify_lm_head_int4_workspace_bytes.argtypes = [i32, i32, i32, i32]
        L.verify_lm_head_int4_workspace_bytes.restype = sz
        L.verify_lm_head_int4_workspace_init.argtypes = [P, sz, P]
        L.verify_lm_head_int4_workspace_init.restype = i32
        L.verify_lm_head_int4.argtypes = [P, P, P, P, i32, i32, i32, P, P, P, P, P, sz, P]
        L.verify_lm_head_int4.restype = i32
        L.verify_lm_head_int4_batch.argtypes = [P, P, P, P, i32, i32, i32, i32, P, P, P, P, P,
                                                sz, P]
        L.verify_lm_head_int4_batch.restype = i32
        L.verify_lm_head_int4_batch_timed.argtypes = [P, P, P, P, i32, i32, i32, i32, P, P, P, P,
                                                      P, sz, P, P, P]
        L.verify_lm_head_int4_batch_timed.restype = i32
        L.verify_lm_head_int4_check_weights.argtypes = [P, i32, i32, P, P]
        L.verify_lm_head_int4_check_weights.restype = i32
        L.verify_lm_head_int4_status_string.argtypes = [i32]
        L.verify_lm_head_int4_status_string.restype = ctypes.c_char_p
        L.verify_lm_head_int4_last_error.argtypes = []
        L.verify_lm_head_int4_last_error.restype = ctypes.c_char_p
        _lib = L
        return L


def _raise(status: int, what: str):
    L = load_library()
    msg = L.verify_lm_head_int4_status_string(status).decode()
    if status == EHIP:
        msg += ": " + L.verify_lm_head_int4_last_error().decode()
    raise RuntimeError(f"{what}: {msg} (status {status})")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_ptr(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def workspace_bytes(R: int, T: int, V: int, H: int) -> int:
    return int(load_library().verify_lm_head_int4_workspace_bytes(R, T, V, H))


class Workspace:
    """A device workspace for verify calls, initialised on creation.  Calls
    that share a Workspace must not be in flight at the same time."""

    def __init__(self, nbytes: int, device):
        self.nbytes = int(nbytes)
        self.tensor = torch.empty(self.nbytes, dtype=torch.uint8, device=device)
        st = load_library().verify_lm_head_int4_workspace_init(
            _ptr(self.tensor), self.nbytes, _stream_ptr(self.tensor.device))
        if st != OK:
            _raise(st, "workspace_init")


_ws_cache: dict = {}


def _default_workspace(device, nbytes: int) -> Workspace:
    # one per (device, current stream): calls on one stream are ordered
    key = (device.index, torch.cuda.current_stream(device).cuda_stream)
    ws = _ws_cache.get(key)
    if ws is None or ws.nbytes < nbytes:
        ws = Workspace(nbytes, device)
        _ws_cache[key] = ws
    return ws


def _check(t, name, dtype, ndim=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {t.dim()}")


def _event_handle(ev, stream):
    """Raw hipEvent_t of a torch.cuda.Event (created by a first record)."""
    if ev.cuda_event == 0:
        ev.record(stream)
    return ctypes.c_void_p(ev.cuda_event)


def verify_batch(hidden, packed_w, scales, draft_ids=None, *, R: int | None = None,
                 logits: bool = False, workspace: Workspace | None = None, events=None):
    """R requests x T positions.  hidden: float16 [R, T, H] (or [R*T, H] with
    R given); packed_w: uint8 [V, H/2]; scales: float16 [H]; draft_ids: int32
    [R, T-1] (None when T == 1).  Returns (logits_max [R*T], argmax_ids [R*T],
    n_accepted [R]) and, with logits=True, logits [R*T, V] as a 4th item.
    events=(before, after), two torch.cuda.Event(enable_timing=True), are
    recorded on the current stream right around the main verify kernel (the
    instrumented entry point verify_lm_head_int4_batch_timed)."""
    if hidden.dim() == 3:
        R, T, H = hidden.shape
        hidden = hidden.reshape(R * T, H)
    else:
        if R is None:
            raise ValueError("R is required for a 2-D hidden tensor")
        T = hidden.shape[0] // R
        H = hidden.shape[1]
    _check(hidden, "hidden", torch.float16, 2)
    _check(packed_w, "packed_w", torch.uint8, 2)
    _check(scales, "scales", torch.float16, 1)
    V = packed_w.shape[0]
    if packed_w.shape[1] * 2 != H or scales.shape[0] != H or hidden.shape[0] != R * T:
        raise ValueError("shape mismatch between hidden, packed_w and scales")
    dev = hidden.device
    if T > 1:
        if draft_ids is None:
            raise ValueError("draft_ids is required when T > 1")
        _check(draft_ids, "draft_ids", torch.int32)
        if draft_ids.numel() != R * (T - 1):
            raise ValueError("draft_ids must hold R*(T-1) ids")
    else:
        draft_ids = None
    M = R * T
    lmax = torch.empty(M, dtype=torch.float32, device=dev)
    amax = torch.empty(M, dtype=torch.int32, device=dev)
    nacc = torch.empty(R, dtype=torch.int32, device=dev)
    lout = torch.empty((M, V), dtype=torch.float32, device=dev) if logits else None
    L = load_library()
    need = L.verify_lm_head_int4_workspace_bytes(R, T, V, H)
    if need == 0:
        _raise(EINVAL, "verify")
    ws = workspace if workspace is not None else _default_workspace(dev, need)
    args = (_ptr(hidden), _ptr(packed_w), _ptr(scales), _ptr(draft_ids), R, T, V, H, _ptr(lmax),
            _ptr(amax), _ptr(nacc), _ptr(lout), _ptr(ws.tensor), ws.nbytes, _stream_ptr(dev))
    if events is None:
        st = L.verify_lm_head_int4_batch(*args)
    else:
        stream = torch.cuda.current_stream(dev)
        st = L.verify_lm_head_int4_batch_timed(*args, _event_handle(events[0], stream),
                                               _event_handle(events[1], stream))
    if st != OK:
        _raise(st, "verify_lm_head_int4_batch")
    return (lmax, amax, nacc, lout) if logits else (lmax, amax, nacc)


def verify(hidden, packed_w, scales, draft_ids=None, *, logits: bool = False,
           workspace: Workspace | None = None):
    """One request.  hidden: float16 [T, H]; draft_ids: int32 [T-1] or None
    when T == 1.  Returns (logits_max [T], argmax_ids [T], n_accepted [1])
    and logits [T, V] with logits=True."""
    _check(hidden, "hidden", torch.float16, 2)
    _check(packed_w, "packed_w", torch.uint8, 2)
    _check(scales, "scales", torch.float16, 1)
    T, H = hidden.shape
    V = packed_w.shape[0]
    if packed_w.shape[1] * 2 != H or scales.shape[0] != H:
        raise ValueError("shape mismatch between hidden, packed_w and scales")
    dev = hidden.device
    if T > 1:
        if draft_ids is None:
            raise ValueError("draft_ids is required when T > 1")
        _check(draft_ids, "draft_ids", torch.int32)
        if draft_ids.numel() != T - 1:
            raise ValueError("draft_ids must hold T-1 ids")
    else:
        draft_ids = None
    lmax = torch.empty(T, dtype=torch.float32, device=dev)
    amax = torch.empty(T, dtype=torch.int32, device=dev)
    nacc = torch.empty(1, dtype=torch.int32, device=dev)
    lout = torch.empty((T, V), dtype=torch.float32, device=dev) if logits else None
    L = load_library()
    need = L.verify_lm_head_int4_workspace_bytes(1, T, V, H)
    if need == 0:
        _raise(EINVAL, "verify")
    ws = workspace if workspace is not None else _default_workspace(dev, need)
    st = L.verify_lm_head_int4(_ptr(hidden), _ptr(packed_w), _ptr(scales), _ptr(draft_ids),
                               T, V, H, _ptr(lmax), _ptr(amax), _ptr(nacc), _ptr(lout),
                               _ptr(ws.tensor), ws.nbytes, _stream_ptr(dev))
    if st != OK:
        _raise(st, "verify_lm_head_int4")
    return (lmax, amax, nacc, lout) if logits else (lmax, amax, nacc)


def check_weights(packed_w) -> torch.Tensor:
    """Number of illegal (0x8) nibbles of a packed head, as an int32 [1]
    device tensor (asynchronous)."""
    _check(packed_w, "packed_w", torch.uint8, 2)
    V, Hh = packed_w.shape
    out = torch.empty(1, dtype=torch.int32, device=packed_w.device)
    st = load_library().verify_lm_head_int4_check_weights(
        _ptr(packed_w), V, 2 * Hh, _ptr(out), _stream_ptr(packed_w.device))
    if st != OK:
        _raise(st, "check_weights")
    return out

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

OK, EINVAL, EALIGN, EWORKSPACE, EHIP, EUNSUPPORTED, ESCRATCH = 0, -1, -2, -3, -4, -5, -6

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
        L.verify_lm_head_int4_sampled_workspace_bytes.argtypes = [i32, i32, i32, i32]
        L.verify_lm_head_int4_sampled_workspace_bytes.restype = sz
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
        L.verify_lm_head_int4_batch_noalloc.argtypes = [P, P, P, P, i32, i32, i32, i32, P, P, P, P,
                                                        P]
        L.verify_lm_head_int4_batch_noalloc.restype = i32
        L.verify_lm_head_int4_check_weights.argtypes = [P, i32, i32, P, P]
        L.verify_lm_head_int4_check_weights.restype = i32
        L.verify_lm_head_int4_status_string.argtypes = [i32]
        L.verify_lm_head_int4_status_string.restype = ctypes.c_char_p
        L.verify_lm_head_int4_last_error.argtypes = []
        L.verify_lm_head_int4_last_error.restype = ctypes.c_char_p
        L.verify_lm_head_int4_mapped.argtypes = [P, P, P, P, P, i32, i32, i32, i32, P, P, P, P,
                                                 P, sz, P]
        L.verify_lm_head_int4_mapped.restype = i32
        L.verify_lm_head_int4_check_vocab_map.argtypes = [P, i32, P, P]
        L.verify_lm_head_int4_check_vocab_map.restype = i32
        L.verify_lm_head_int4_sampled.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, i32,
                                                  ctypes.c_float, P, P, P, P, P, P, P, P, sz, P]
        L.verify_lm_head_int4_sampled.restype = i32
        L.verify_lm_head_int4_sampled_timed.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, i32,
                                                        ctypes.c_float, P, P, P, P, P, P, P, P, sz,
                                                        P, P, P]
        L.verify_lm_head_int4_sampled_timed.restype = i32
        # read-only streaming reference (include/int4vh_probe.h)
        L.int4vh_stream_read.argtypes = [P, sz, i32, P, P, P, P]
        L.int4vh_stream_read.restype = i32
        # context-copy drafter (include/int4vh_drafter.h)
        L.context_copy_propose.argtypes = [P, P, i32, P, i32, i32, i32, P, P, P, P, P]
        L.context_copy_propose.restype = i32
        L.context_copy_propose_timed.argtypes = [P, P, i32, P, i32, i32, i32, P, P, P, P, P, P, P]
        L.context_copy_propose_timed.restype = i32
        # offline requantisation (include/int4vh_requant.h)
        L.requant_lm_head_int4_amax.argtypes = [P, i32, i32, i32, P, i32, P]
        L.requant_lm_head_int4_amax.restype = i32
        L.requant_lm_head_int4_scales.argtypes = [P, i32, P, P]
        L.requant_lm_head_int4_scales.restype = i32
        L.requant_lm_head_int4_pack.argtypes = [P, i32, i32, i32, P, P, P]
        L.requant_lm_head_int4_pack.restype = i32
        L.requant_lm_head_int4_pack_timed.argtypes = [P, i32, i32, i32, P, P, P, P, P]
        L.requant_lm_head_int4_pack_timed.restype = i32
        L.requant_lm_head_int4.argtypes = [P, i32, i32, i32, P, i32, i32, P, P, P, P]
        L.requant_lm_head_int4.restype = i32
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


def sampled_workspace_bytes(R: int, T: int, V: int, H: int) -> int:
    return int(load_library().verify_lm_head_int4_sampled_workspace_bytes(R, T, V, H))


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
    """Raw hipEvent_t of a torch.cuda.Event (created by a first record);
    None gives a null handle (that end of the kernel is not timed)."""
    if ev is None:
        return ctypes.c_void_p(None)
    if ev.cuda_event == 0:
        ev.record(stream)
    return ctypes.c_void_p(ev.cuda_event)


def verify_batch(hidden, packed_w, scales, draft_ids=None, *, R: int | None = None,
                 logits: bool = False, workspace: Workspace | None = None, events=None):
    """R requests x T positions.  hidden: float16 [R, T, H] (or [R*T, H] with
    R given); packed_w: uint8 [V, H/2]; scales: float16 [H]; draft_ids: int32
    [R, T-1] (None when T == 1).  Returns (logits_max [R*T], argmax_ids [R*T],
    n_accepted [R]) and, with logits=True, logits [R*T, V] as a 4th item.
    events=(before, after), two torch.cuda.Event(enable_timing=True), take
    the start and end timestamps of the main verify kernel's own dispatch
    (the instrumented entry point verify_lm_head_int4_batch_timed; not for
    use under graph capture)."""
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


def verify_batch_noalloc(hidden, packed_w, scales, draft_ids=None, *, R: int | None = None,
                         logits: bool = False, out=None):
    """verify_batch through the entry point that allocates nothing
    (verify_lm_head_int4_batch_noalloc: the library's static per-device
    scratch replaces the workspace).  out=(logits_max, argmax_ids,
    n_accepted[, logits]) supplies preallocated outputs (as a caller under
    graph capture would); otherwise they are allocated here, by torch.  Calls
    that overlap in time on one device race on the shared scratch."""
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
    if out is not None:
        lmax, amax, nacc = out[0], out[1], out[2]
        lout = out[3] if len(out) > 3 else None
        _check(lmax, "logits_max", torch.float32)
        _check(amax, "argmax_ids", torch.int32)
        _check(nacc, "n_accepted", torch.int32)
        if lmax.numel() != M or amax.numel() != M or nacc.numel() != R:
            raise ValueError("output sizes do not match R*T rows and R requests")
        if lout is not None:
            _check(lout, "logits", torch.float32)
            if lout.numel() != M * V:
                raise ValueError("logits must hold R*T*V values")
    else:
        lmax = torch.empty(M, dtype=torch.float32, device=dev)
        amax = torch.empty(M, dtype=torch.int32, device=dev)
        nacc = torch.empty(R, dtype=torch.int32, device=dev)
        lout = torch.empty((M, V), dtype=torch.float32, device=dev) if logits else None
    st = load_library().verify_lm_head_int4_batch_noalloc(
        _ptr(hidden), _ptr(packed_w), _ptr(scales), _ptr(draft_ids), R, T, V, H, _ptr(lmax),
        _ptr(amax), _ptr(nacc), _ptr(lout), _stream_ptr(dev))
    if st != OK:
        _raise(st, "verify_batch_noalloc")
    return (lmax, amax, nacc, lout) if lout is not None else (lmax, amax, nacc)


def verify_mapped(hidden, packed_w, scales, vocab_ids, draft_ids=None, *, R: int | None = None,
                  logits: bool = False, workspace: Workspace | None = None):
    """Verify through a head whose rows are a subset of the vocabulary:
    vocab_ids (int32 [V], strictly increasing) maps each head row to its
    token id; argmax_ids are token ids and draft_ids are compared with them.
    Otherwise as verify_batch (hidden [R, T, H], or [R*T, H] with R)."""
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
    _check(vocab_ids, "vocab_ids", torch.int32, 1)
    V = packed_w.shape[0]
    if packed_w.shape[1] * 2 != H or scales.shape[0] != H or hidden.shape[0] != R * T:
        raise ValueError("shape mismatch between hidden, packed_w and scales")
    if vocab_ids.shape[0] != V:
        raise ValueError("vocab_ids must hold one id per head row")
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
        _raise(EINVAL, "verify_mapped")
    ws = workspace if workspace is not None else _default_workspace(dev, need)
    st = L.verify_lm_head_int4_mapped(_ptr(hidden), _ptr(packed_w), _ptr(scales), _ptr(vocab_ids),
                                      _ptr(draft_ids), R, T, V, H, _ptr(lmax), _ptr(amax), _ptr(nacc),
                                      _ptr(lout), _ptr(ws.tensor), ws.nbytes, _stream_ptr(dev))
    if st != OK:
        _raise(st, "verify_lm_head_int4_mapped")
    return (lmax, amax, nacc, lout) if logits else (lmax, amax, nacc)


def verify_sampled(hidden, packed_w, scales, draft_ids=None, draft_probs=None, uniforms=None, *,
                   top_k: int, temperature: float = 1.0, R: int | None = None,
                   workspace: Workspace | None = None, events=None, want_lse: bool = False):
    """Sampled verification for R*T <= 4096 rows: top-k sampling at a
    temperature (top_k >= 1) or sampling over the whole vocabulary
    (top_k == 0).  hidden: float16 [R, T, H] (or [R*T, H] with R); draft_ids
    int32, draft_probs and uniforms float32, each [R, T-1] (None when T == 1).
    Returns (logits_max [R*T], argmax_ids [R*T], topk_ids [R*T, k],
    topk_logits [R*T, k], p_draft [R, T-1], n_accepted [R], lse [R*T]) (the
    top-k outputs are None when top_k == 0; lse, the log-sum-exp of
    logit / temperature over the vocabulary, is None unless want_lse or
    top_k == 0).  events=(before, after) take the start and end timestamps of
    the main verify kernel's dispatch.  Above 64 rows the workspace also
    holds the call's logits (sampled_workspace_bytes)."""
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
        for t, n, dt in ((draft_ids, "draft_ids", torch.int32), (draft_probs, "draft_probs", torch.float32),
                         (uniforms, "uniforms", torch.float32)):
            if t is None:
                raise ValueError(f"{n} is required when T > 1")
            _check(t, n, dt)
            if t.numel() != R * (T - 1):
                raise ValueError(f"{n} must hold R*(T-1) values")
    else:
        draft_ids = draft_probs = uniforms = None
    M = R * T
    k = int(top_k)
    lmax = torch.empty(M, dtype=torch.float32, device=dev)
    amax = torch.empty(M, dtype=torch.int32, device=dev)
    tids = torch.empty((M, k), dtype=torch.int32, device=dev) if k > 0 else None
    tlog = torch.empty((M, k), dtype=torch.float32, device=dev) if k > 0 else None
    lse = torch.empty(M, dtype=torch.float32, device=dev) if (want_lse or k == 0) else None
    pdr = torch.empty((R, max(T - 1, 1)), dtype=torch.float32, device=dev)
    nacc = torch.empty(R, dtype=torch.int32, device=dev)
    L = load_library()
    need = L.verify_lm_head_int4_sampled_workspace_bytes(R, T, V, H)
    if need == 0:
        _raise(EINVAL, "verify_sampled")
    ws = workspace if workspace is not None else _default_workspace(dev, need)
    args = (_ptr(hidden), _ptr(packed_w), _ptr(scales), _ptr(draft_ids), _ptr(draft_probs),
            _ptr(uniforms), R, T, V, H, k, float(temperature), _ptr(lmax), _ptr(amax), _ptr(tids),
            _ptr(tlog), _ptr(lse), _ptr(pdr), _ptr(nacc), _ptr(ws.tensor), ws.nbytes, _stream_ptr(dev))
    if events is None:
        st = L.verify_lm_head_int4_sampled(*args)
    else:
        stream = torch.cuda.current_stream(dev)
        st = L.verify_lm_head_int4_sampled_timed(*args, _event_handle(events[0], stream),
                                                 _event_handle(events[1], stream))
    if st != OK:
        _raise(st, "verify_lm_head_int4_sampled")
    return lmax, amax, tids, tlog, pdr[:, : max(T - 1, 0)], nacc, lse


def check_vocab_map(vocab_ids) -> torch.Tensor:
    """Number of positions where vocab_ids is not strictly increasing and
    non-negative, as an int32 [1] device tensor (asynchronous)."""
    _check(vocab_ids, "vocab_ids", torch.int32, 1)
    out = torch.empty(1, dtype=torch.int32, device=vocab_ids.device)
    st = load_library().verify_lm_head_int4_check_vocab_map(
        _ptr(vocab_ids), vocab_ids.shape[0], _ptr(out), _stream_ptr(vocab_ids.device))
    if st != OK:
        _raise(st, "check_vocab_map")
    return out


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


# ---------------------------------------------------------------- requantisation

F16, BF16 = 0, 1
_DTYPES = {torch.float16: F16, torch.bfloat16: BF16}


def _dtype_code(t, name):
    if t.dtype not in _DTYPES:
        raise TypeError(f"{name} must be float16 or bfloat16, got {t.dtype}")
    return _DTYPES[t.dtype]


def requant_amax(acts, amax=None, *, accumulate: bool = False) -> torch.Tensor:
    """Per-channel max |acts| of calibration rows acts [N, H] (float16 or
    bfloat16) into amax (float32 [H]); with accumulate=True the running
    maximum of an existing amax.  Returns amax (asynchronous)."""
    if not isinstance(acts, torch.Tensor) or not acts.is_cuda:
        raise TypeError("acts must be a CUDA (HIP) tensor")
    dt = _dtype_code(acts, "acts")
    _check(acts, "acts", acts.dtype, 2)
    N, H = acts.shape
    if amax is None:
        if accumulate:
            raise ValueError("accumulate=True needs an existing amax")
        amax = torch.empty(H, dtype=torch.float32, device=acts.device)
    _check(amax, "amax", torch.float32, 1)
    if amax.shape[0] != H:
        raise ValueError("amax must hold H values")
    st = load_library().requant_lm_head_int4_amax(_ptr(acts), dt, N, H, _ptr(amax), int(accumulate),
                                                  _stream_ptr(acts.device))
    if st != OK:
        _raise(st, "requant_lm_head_int4_amax")
    return amax


def requant_scales(amax) -> torch.Tensor:
    """float16 scales [H] = amax / 7 (binary32 division, rounded to binary16)."""
    _check(amax, "amax", torch.float32, 1)
    H = amax.shape[0]
    scales = torch.empty(H, dtype=torch.float16, device=amax.device)
    st = load_library().requant_lm_head_int4_scales(_ptr(amax), H, _ptr(scales),
                                                    _stream_ptr(amax.device))
    if st != OK:
        _raise(st, "requant_lm_head_int4_scales")
    return scales


def requant_pack(W, scales, *, events=None) -> torch.Tensor:
    """Quantise the head W [V, H] (float16 or bfloat16) with per-channel
    scales (float16 [H]) and pack it: uint8 [V, H/2] in the verify layout.
    events=(before, after) take the start and end timestamps of the pack
    kernel's dispatch."""
    if not isinstance(W, torch.Tensor) or not W.is_cuda:
        raise TypeError("W must be a CUDA (HIP) tensor")
    dt = _dtype_code(W, "W")
    _check(W, "W", W.dtype, 2)
    _check(scales, "scales", torch.float16, 1)
    V, H = W.shape
    if scales.shape[0] != H:
        raise ValueError("scales must hold H values")
    packed = torch.empty((V, H // 2), dtype=torch.uint8, device=W.device)
    L = load_library()
    if events is None:
        st = L.requant_lm_head_int4_pack(_ptr(W), dt, V, H, _ptr(scales), _ptr(packed),
                                         _stream_ptr(W.device))
    else:
        stream = torch.cuda.current_stream(W.device)
        st = L.requant_lm_head_int4_pack_timed(_ptr(W), dt, V, H, _ptr(scales), _ptr(packed),
                                               _stream_ptr(W.device),
                                               _event_handle(events[0], stream),
                                               _event_handle(events[1], stream))
    if st != OK:
        _raise(st, "requant_lm_head_int4_pack")
    return packed


def requantize(W, acts):
    """The whole offline step for one calibration batch: returns (packed
    uint8 [V, H/2], scales float16 [H], amax float32 [H])."""
    for t, n in ((W, "W"), (acts, "acts")):
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise TypeError(f"{n} must be a CUDA (HIP) tensor")
    wdt, adt = _dtype_code(W, "W"), _dtype_code(acts, "acts")
    _check(W, "W", W.dtype, 2)
    _check(acts, "acts", acts.dtype, 2)
    V, H = W.shape
    N = acts.shape[0]
    if acts.shape[1] != H:
        raise ValueError("acts and W must have the same H")
    dev = W.device
    amax = torch.empty(H, dtype=torch.float32, device=dev)
    scales = torch.empty(H, dtype=torch.float16, device=dev)
    packed = torch.empty((V, H // 2), dtype=torch.uint8, device=dev)
    st = load_library().requant_lm_head_int4(_ptr(W), wdt, V, H, _ptr(acts), adt, N, _ptr(amax),
                                             _ptr(scales), _ptr(packed), _stream_ptr(dev))
    if st != OK:
        _raise(st, "requant_lm_head_int4")
    return packed, scales, amax


# ---------------------------------------------------------------- context-copy drafter

def context_copy(prompts, offsets, keys, *, n_min: int = 1, n_out: int = 8, events=None):
    """Propose the tokens copied from each request's prompt.  prompts: int32
    [total] (all prompts back to back); offsets: int64 [R+1]; keys: int32
    [R, n_max] (the last n_max tokens of each sequence).  Returns (tokens
    int32 [R, n_out] (-1 past count), count [R], match_end [R], match_len
    [R]).  events=(before, after) take the kernel's dispatch start and end."""
    _check(prompts, "prompts", torch.int32, 1)
    _check(offsets, "offsets", torch.int64, 1)
    _check(keys, "keys", torch.int32, 2)
    R, n_max = keys.shape
    if offsets.shape[0] != R + 1:
        raise ValueError("offsets must hold R+1 values")
    dev = prompts.device
    tok = torch.empty((R, n_out), dtype=torch.int32, device=dev)
    cnt = torch.empty(R, dtype=torch.int32, device=dev)
    end = torch.empty(R, dtype=torch.int32, device=dev)
    ln = torch.empty(R, dtype=torch.int32, device=dev)
    L = load_library()
    args = (_ptr(prompts), _ptr(offsets), R, _ptr(keys), n_max, n_min, n_out, _ptr(tok), _ptr(cnt),
            _ptr(end), _ptr(ln), _stream_ptr(dev))
    if events is None:
        st = L.context_copy_propose(*args)
    else:
        stream = torch.cuda.current_stream(dev)
        st = L.context_copy_propose_timed(*args, _event_handle(events[0], stream),
                                          _event_handle(events[1], stream))
    if st != OK:
        _raise(st, "context_copy_propose")
    return tok, cnt, end, ln


PROBE_OUT_WORDS = 8192


def stream_read(buf, mode: int = 0, *, out=None, events=None):
    """Read the device tensor `buf` once (int4vh_stream_read): mode 0 loads
    into registers, mode 1 copies into LDS like the verify kernel.  Returns
    the per-wave words (uint32 as int32 [8192]); in mode 0 their xor is the
    xor of the buffer's 32-bit words.  events=(before, after) take the
    kernel's dispatch start and end."""
    if not isinstance(buf, torch.Tensor) or not buf.is_cuda or not buf.is_contiguous():
        raise TypeError("buf must be a contiguous CUDA (HIP) tensor")
    dev = buf.device
    if out is None:
        out = torch.zeros(PROBE_OUT_WORDS, dtype=torch.int32, device=dev)
    nbytes = buf.numel() * buf.element_size()
    stream = torch.cuda.current_stream(dev)
    e0 = _event_handle(events[0], stream) if events else None
    e1 = _event_handle(events[1], stream) if events else None
    st = load_library().int4vh_stream_read(_ptr(buf), nbytes, int(mode), _ptr(out), _stream_ptr(dev), e0, e1)
    if st != OK:
        _raise(st, "int4vh_stream_read")
    return out

"""The entry point that allocates nothing (verify_lm_head_int4_batch_noalloc)
against the workspace entry point it mirrors (verify_lm_head_int4_batch).

Both run the same kernels, so every output must be identical bit for bit.
The no-allocation call keeps its workspace in one static scratch array per
device, shared by every call: consecutive calls of different sizes (largest
first, so a later call runs over what an earlier one left behind), a call at
the full-vocabulary T = 16 shape, and graph replays interleaved with eager
calls must all match.  The size limit is checked on the host (no GPU).
"""
import ctypes
import os
import sys

import numpy as np
import pytest

from int4_output_head_amd import synth

from . import parity

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "int4_output_head_amd", "libint4vh.so")
ESCRATCH = -6
SCRATCH_BYTES = 16 << 20


def say(msg):
    print(f"[no-alloc] {msg}", flush=True)
    sys.stdout.flush()


def _lib():
    if not os.path.exists(LIB):
        from int4_output_head_amd.build import build_library
        build_library()
    L = ctypes.CDLL(LIB)
    P, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    L.verify_lm_head_int4_batch_noalloc.argtypes = [P, P, P, P, i32, i32, i32, i32, P, P, P, P, P]
    L.verify_lm_head_int4_batch_noalloc.restype = i32
    L.verify_lm_head_int4_workspace_bytes.argtypes = [i32, i32, i32, i32]
    L.verify_lm_head_int4_workspace_bytes.restype = sz
    return L


def test_noalloc_scratch_limit_on_host():
    """Shapes whose workspace exceeds the 16 MiB scratch return
    INT4VH_ESCRATCH before any GPU call (fake, never-dereferenced pointers);
    invalid arguments still return their usual codes first."""
    L = _lib()
    fake = ctypes.c_void_p(1 << 20)
    args = lambda R, T, V, H: (fake, fake, fake, fake if T > 1 else None, R, T, V, H, fake, fake, fake,
                               None, None)
    # 1024 rows at H = 5120 fit, 1025 do not
    assert L.verify_lm_head_int4_workspace_bytes(1024, 1, 151936, 5120) <= SCRATCH_BYTES
    assert L.verify_lm_head_int4_workspace_bytes(1025, 1, 151936, 5120) > SCRATCH_BYTES
    assert L.verify_lm_head_int4_batch_noalloc(*args(1025, 1, 151936, 5120)) == ESCRATCH
    assert L.verify_lm_head_int4_batch_noalloc(*args(1024, 4, 151936, 5120)) == ESCRATCH
    assert L.verify_lm_head_int4_batch_noalloc(*args(1, 17, 100, 64)) == -1        # T > 16
    assert L.verify_lm_head_int4_batch_noalloc(*args(1, 4, 100, 48)) == -1         # H % 32
    bad = (fake, fake, fake, fake, 1, 4, 100, 64, ctypes.c_void_p((1 << 20) + 4), fake, fake, None, None)
    assert L.verify_lm_head_int4_batch_noalloc(*bad) == -2                         # misaligned


torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def vh():
    from int4_output_head_amd import binding
    binding.load_library()
    assert torch.cuda.is_available(), "no GPU visible"
    return binding


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.cuda()


def noalloc(hidden, packed, scales, drafts, R, T, V, H, logits=True):
    """One call of the C entry point with torch-allocated outputs."""
    L = _lib()
    M = R * T
    lmax = torch.empty(M, dtype=torch.float32, device="cuda")
    amax = torch.empty(M, dtype=torch.int32, device="cuda")
    nacc = torch.empty(R, dtype=torch.int32, device="cuda")
    lout = torch.empty((M, V), dtype=torch.float32, device="cuda") if logits else None
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    st = L.verify_lm_head_int4_batch_noalloc(
        p(hidden), p(packed), p(scales), p(drafts), R, T, V, H, p(lmax), p(amax), p(nacc), p(lout),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, st
    return (lmax, amax, nacc, lout) if logits else (lmax, amax, nacc)


def reference(vh, hidden, packed, scales, drafts, R, logits=True):
    """The workspace entry point, on a fresh workspace of its own."""
    T = hidden.shape[0] // R
    ws = vh.Workspace(vh.workspace_bytes(R, T, packed.shape[0], hidden.shape[1]), hidden.device)
    return vh.verify_batch(hidden, packed, scales, drafts, R=R, logits=logits, workspace=ws)


def inputs(R, T, V, H, seed):
    d = synth.uniform_inputs(R * T, V, H, seed=seed)
    rng = np.random.default_rng(seed)
    drafts = rng.integers(0, V, size=(R, T - 1)).astype(np.int32) if T > 1 else None
    return d, drafts


@pytest.mark.gpu
def test_noalloc_matches_batch_consecutive_calls(vh, oracle_mod):
    """Three calls in a row, each smaller than the one before: 64 rows (the
    batch kernels), 16 rows, 2 rows (staging inside the verify kernel); all
    identical to the workspace entry point, the first also against the
    oracle."""
    for i, (R, T, V, H) in enumerate([(16, 4, 3001, 640), (2, 8, 2000, 512), (1, 2, 1000, 256)]):
        say(f"call {i}: R={R} T={T} V={V} H={H}")
        d, dr = inputs(R, T, V, H, seed=100 + i)
        if dr is not None:
            # drafts that follow the oracle argmax for a while, so acceptance counts are nonzero
            o = oracle_mod.verify(d["hidden"], d["packed"], d["scales"], dr, R, T, V, H, want_logits=True)
            dr[:, : (T - 1) // 2] = o["argmax_ids"].reshape(R, T)[:, : (T - 1) // 2]
        o = oracle_mod.verify(d["hidden"], d["packed"], d["scales"], dr, R, T, V, H, want_logits=True)
        x, w, s = dev(d["hidden"], torch.float16), dev(d["packed"]), dev(d["scales"], torch.float16)
        dt = dev(dr) if dr is not None else None
        got = noalloc(x, w, s, dt, R, T, V, H)
        ref = reference(vh, x, w, s, dt, R)
        torch.cuda.synchronize()
        for a, b in zip(got, ref):
            assert torch.equal(a, b)
        g = dict(logits_max=got[0].cpu().numpy(), argmax_ids=got[1].cpu().numpy(),
                 n_accepted=got[2].cpu().numpy(), logits=got[3].cpu().numpy())
        stats = parity.check(g, o, R, T, dr)
        say(f"call {i}: equal to the workspace entry point; oracle {stats}")


@pytest.mark.gpu
def test_noalloc_full_vocab_t16(vh):
    """The full-vocabulary T = 16 verify block, then a 1-row call."""
    cfg = synth.CONFIGS["full_t16"]
    head = synth.make_head(cfg)
    w, s = dev(head["packed"]), dev(head["scales"], torch.float16)
    for T in (16, 1):
        x = dev(synth.make_hidden(cfg, 3)[:T], torch.float16)
        dt = dev(np.arange(T - 1, dtype=np.int32)) if T > 1 else None
        got = noalloc(x, w, s, dt, 1, T, cfg.V, cfg.H, logits=False)
        ref = reference(vh, x, w, s, dt, 1, logits=False)
        torch.cuda.synchronize()
        for a, b in zip(got, ref):
            assert torch.equal(a, b)
        say(f"full vocabulary T={T}: equal to the workspace entry point")


@pytest.mark.gpu
def test_noalloc_graph_replays(vh):
    """Captured in a HIP graph with preallocated outputs, replayed three
    times with eager no-allocation calls of another shape in between (which
    rewrite the shared scratch); every replay equals the eager result."""
    R, T, V, H = 1, 8, 5000, 512
    d, dr = inputs(R, T, V, H, seed=7)
    x, w, s, dt = dev(d["hidden"], torch.float16), dev(d["packed"]), dev(d["scales"], torch.float16), dev(dr)
    d2, dr2 = inputs(4, 8, 2500, 256, seed=8)
    x2, w2, s2, dt2 = dev(d2["hidden"], torch.float16), dev(d2["packed"]), dev(d2["scales"], torch.float16), \
        dev(dr2)
    want = noalloc(x, w, s, dt, R, T, V, H, logits=False)
    torch.cuda.synchronize()
    out = (torch.empty(R * T, dtype=torch.float32, device="cuda"),
           torch.empty(R * T, dtype=torch.int32, device="cuda"),
           torch.empty(R, dtype=torch.int32, device="cuda"))
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        vh.verify_batch_noalloc(x, w, s, dt, R=R, out=out)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=stream):
            vh.verify_batch_noalloc(x, w, s, dt, R=R, out=out)
    torch.cuda.synchronize()
    for rep in range(3):
        for o in out:
            o.fill_(-1)
        other = noalloc(x2, w2, s2, dt2, 4, 8, 2500, 256, logits=False)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(out, want):
            assert torch.equal(a, b), rep
        ref2 = reference(vh, x2, w2, s2, dt2, 4, logits=False)
        torch.cuda.synchronize()
        for a, b in zip(other, ref2):
            assert torch.equal(a, b), rep
        say(f"replay {rep}: equal to the eager call")

"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.  Needs an MI355X and the built library."""
import os
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from int4_output_head_amd import synth  # noqa: E402

from . import parity  # noqa: E402

pytestmark = pytest.mark.gpu

NTHREADS = min(16, os.cpu_count() or 1)


def say(msg):
    print(f"[gpu-parity] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def vh():
    from int4_output_head_amd import binding
    binding.load_library()
    assert torch.cuda.is_available(), "no GPU visible"
    return binding


@pytest.fixture(scope="module")
def orc(oracle_mod):
    return oracle_mod


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.cuda()


def run_gpu(vh, hidden_bits, packed, scales_bits, drafts, R, T, logits=True, packed_dev=None):
    x = dev(hidden_bits, torch.float16)
    w = packed_dev if packed_dev is not None else dev(packed)
    s = dev(scales_bits, torch.float16)
    d = None if T == 1 else dev(np.asarray(drafts, np.int32).reshape(R, T - 1))
    out = vh.verify_batch(x.reshape(R, T, -1), w, s, d, logits=logits)
    torch.cuda.synchronize()
    res = dict(logits_max=out[0].cpu().numpy(), argmax_ids=out[1].cpu().numpy(),
               n_accepted=out[2].cpu().numpy())
    if logits:
        res["logits"] = out[3].cpu().numpy()
    return res


def oracle_case(orc, hidden_bits, packed, scales_bits, drafts, R, T, V, H):
    return orc.verify(hidden_bits, packed, scales_bits, drafts, R, T, V, H, want_logits=True,
                      n_threads=NTHREADS)


def drafts_for(cfg, trial, oracle_argmax):
    return synth.finalize_drafts(cfg, synth.draft_plan(cfg, trial), oracle_argmax)


# ------------------------------------------------------------------ the configs

def test_tiny_config(vh, orc):
    cfg = synth.CONFIGS["tiny"]
    head = synth.make_head(cfg)
    x = synth.make_hidden(cfg, 0)
    o0 = orc.verify(x, head["packed"], head["scales"], np.zeros(cfg.T - 1, np.int32), 1, cfg.T,
                    cfg.V, cfg.H, n_threads=NTHREADS)
    drafts = drafts_for(cfg, 0, o0["argmax_ids"])
    o = oracle_case(orc, x, head["packed"], head["scales"], drafts, 1, cfg.T, cfg.V, cfg.H)
    say(f"tiny V={cfg.V} H={cfg.H} T={cfg.T}")
    g = run_gpu(vh, x, head["packed"], head["scales"], drafts, 1, cfg.T)
    st = parity.check(g, o, 1, cfg.T, drafts)
    say(f"tiny stats {st}")
    assert o["n_accepted"][0] >= 2


def test_draft_vocab_config(vh, orc):
    cfg = synth.CONFIGS["draft_vocab"]
    head = synth.make_head(cfg)
    w = dev(head["packed"])
    for trial in range(8):
        x = synth.make_hidden(cfg, trial)
        o = oracle_case(orc, x, head["packed"], head["scales"], None, 1, 1, cfg.V, cfg.H)
        say(f"draft_vocab trial {trial}")
        g = run_gpu(vh, x, head["packed"], head["scales"], None, 1, 1, packed_dev=w)
        parity.check(g, o, 1, 1, None)
        assert g["n_accepted"][0] == 0


@pytest.fixture(scope="module")
def full_head():
    cfg = synth.CONFIGS["full_t16"]
    head = synth.make_head(cfg)
    return head, dev(head["packed"])


@pytest.mark.parametrize("name,trial,with_logits", [("full_t8", 0, True), ("full_t16", 0, True),
                                                    ("full_t16", 1, False)])
def test_full_vocab_configs(vh, orc, full_head, name, trial, with_logits):
    cfg = synth.CONFIGS[name]
    head, w = full_head
    x = synth.make_hidden(cfg, trial)
    lg = orc.logits(x, head["packed"], head["scales"], cfg.M, cfg.V, cfg.H, n_threads=NTHREADS)
    idx, mx, gap, amax = orc.argmax_rows(lg)
    drafts = drafts_for(cfg, trial, idx)
    o = dict(logits=lg, logits_max=mx, argmax_ids=idx, gap=gap, amax=amax,
             n_accepted=orc.accept(idx, drafts, cfg.R, cfg.T))
    say(f"{name} trial {trial} logits={with_logits}")
    g = run_gpu(vh, x, head["packed"], head["scales"], drafts, cfg.R, cfg.T, logits=with_logits,
                packed_dev=w)
    st = parity.check(g, o, cfg.R, cfg.T, drafts, orc_logit_at=lambda r, v: float(lg[r, v]))
    say(f"{name} stats {st}")


# ------------------------------------------------------------------ exact mode

@pytest.mark.parametrize("M,V,H", [(4, 300, 128), (16, 1000, 512), (8, 4097, 5120),
                                   (1, 33, 32), (13, 2048, 2080)])
def test_int_exact_bitexact(vh, orc, M, V, H):
    d = synth.int_exact_inputs(M, V, H, seed=M + V + H)
    R, T = 1, M
    o0 = orc.verify(d["hidden"], d["packed"], d["scales"], np.zeros(max(T - 1, 0), np.int32),
                    R, T, V, H, want_logits=True, n_threads=NTHREADS)
    drafts = o0["argmax_ids"][: T - 1].copy()
    if T > 3:
        drafts[T // 2] = (drafts[T // 2] + 1) % V
    o = oracle_case(orc, d["hidden"], d["packed"], d["scales"], drafts, R, T, V, H)
    say(f"int-exact M={M} V={V} H={H}")
    g = run_gpu(vh, d["hidden"], d["packed"], d["scales"], drafts, R, T)
    assert np.array_equal(g["logits"], o["logits"])
    assert np.array_equal(g["argmax_ids"], o["argmax_ids"])
    assert np.array_equal(g["logits_max"], o["logits_max"])
    assert np.array_equal(g["n_accepted"], o["n_accepted"])


def test_int_exact_full_vocab(vh, orc):
    M, V, H = 16, 151936, 5120
    d = synth.int_exact_inputs(M, V, H, seed=99)
    lg = orc.logits(d["hidden"], d["packed"], d["scales"], M, V, H, n_threads=NTHREADS)
    idx, mx, _, _ = orc.argmax_rows(lg)
    drafts = idx[: M - 1].copy()
    drafts[11] = -5
    say("int-exact full vocab M=16")
    g = run_gpu(vh, d["hidden"], d["packed"], d["scales"], drafts, 1, M)
    assert np.array_equal(g["logits"], lg)
    assert np.array_equal(g["argmax_ids"], idx)
    assert np.array_equal(g["logits_max"], mx)
    assert g["n_accepted"][0] == 11


def test_ties_across_tiles(vh, orc):
    """Copies of one row at several indices (same tile, other tiles, last
    tile, other workgroups' tiles): the lowest index must win."""
    M, V, H = 3, 20000, 256
    d = synth.int_exact_inputs(M, V, H, seed=5)
    q = d["q"].copy()
    q[:, :] = np.clip(q, -3, 3)
    best = np.full(H, 7, np.int8)
    for v in (19999, 12345, 4100, 17, 16, 5):
        q[v] = best
    x = np.abs(d["hidden"].view(np.float16).astype(np.float64))  # nonnegative: row of 7s wins
    xb = synth.f16_bits(x)
    packed = synth.pack_int4(q)
    o = oracle_case(orc, xb, packed, d["scales"], np.array([5, 5], np.int32), 1, M, V, H)
    assert np.all(o["argmax_ids"][o["amax"] > 0] == 5)
    say("ties across tiles")
    g = run_gpu(vh, xb, packed, d["scales"], np.array([5, 5], np.int32), 1, M)
    assert np.array_equal(g["argmax_ids"], o["argmax_ids"])
    assert np.array_equal(g["logits"], o["logits"])
    assert g["n_accepted"][0] == o["n_accepted"][0]


# ------------------------------------------------------------------ shapes and edge cases

FUZZ = [(1, 1, 32), (1, 15, 64), (2, 16, 32), (3, 17, 96), (4, 4095, 256), (5, 8193, 2048),
        (7, 257, 5120), (8, 16, 5120), (9, 1, 64), (10, 17, 160), (11, 4095, 1024),
        (12, 8193, 256), (13, 100, 8192), (14, 31, 6144), (15, 512, 4096), (16, 1, 32),
        (16, 15, 5120), (16, 8193, 5120), (8, 70000, 64), (6, 3, 7168), (2, 5000, 8160)]


@pytest.mark.parametrize("T,V,H", FUZZ)
def test_shape_fuzz(vh, orc, T, V, H):
    d = synth.uniform_inputs(T, V, H, seed=T * 7919 + V + H, heavy_frac=0.05)
    o0 = orc.verify(d["hidden"], d["packed"], d["scales"], np.zeros(max(T - 1, 0), np.int32), 1, T,
                    V, H, n_threads=NTHREADS)
    drafts = o0["argmax_ids"][: T - 1].copy()
    if T > 2:
        drafts[T - 2] = V + 3  # out-of-range id never matches
    o = oracle_case(orc, d["hidden"], d["packed"], d["scales"], drafts, 1, T, V, H)
    say(f"fuzz T={T} V={V} H={H}")
    g = run_gpu(vh, d["hidden"], d["packed"], d["scales"], drafts, 1, T)
    parity.check(g, o, 1, T, drafts)


def test_zero_scales(vh, orc):
    T, V, H = 5, 999, 256
    d = synth.uniform_inputs(T, V, H, seed=1)
    s0 = np.zeros(H, np.uint16)
    drafts = np.array([0, 0, 0, 7], np.int32)
    say("zero scales")
    g = run_gpu(vh, d["hidden"], d["packed"], s0, drafts, 1, T)
    assert np.all(g["logits"] == 0) and not np.any(np.signbit(g["logits"]))
    assert np.all(g["argmax_ids"] == 0) and np.all(g["logits_max"] == 0)
    assert g["n_accepted"][0] == 3


def test_one_hot_and_subnormal_hidden(vh, orc):
    T, V, H = 4, 3000, 512
    d = synth.uniform_inputs(T, V, H, seed=2)
    x = np.zeros((T, H))
    x[0, 3] = 1.0
    x[1, 511] = -2.0
    x[2, 100] = 2.0 ** -20       # binary16 subnormal
    x[3] = d["hidden"][3].view(np.float16).astype(np.float64)
    x[3, :40] = 2.0 ** -24        # smallest binary16 subnormal
    xb = synth.f16_bits(x)
    o = oracle_case(orc, xb, d["packed"], d["scales"], np.zeros(3, np.int32), 1, T, V, H)
    say("one-hot and subnormal hidden")
    g = run_gpu(vh, xb, d["packed"], d["scales"], np.zeros(3, np.int32), 1, T)
    # one-hot rows are exact: a single product per logit
    assert np.array_equal(g["logits"][:3], o["logits"][:3])
    assert np.array_equal(g["argmax_ids"][:3], o["argmax_ids"][:3])
    parity.check(g, o, 1, T, np.zeros(3, np.int32))


def test_determinism(vh, orc):
    T, V, H = 16, 40000, 5120
    d = synth.uniform_inputs(T, V, H, seed=3, heavy_frac=0.05)
    drafts = np.arange(T - 1, dtype=np.int32)
    say("determinism")
    a = run_gpu(vh, d["hidden"], d["packed"], d["scales"], drafts, 1, T)
    b = run_gpu(vh, d["hidden"], d["packed"], d["scales"], drafts, 1, T)
    for k in a:
        assert np.array_equal(a[k], b[k]), k
    c = run_gpu(vh, d["hidden"], d["packed"], d["scales"], drafts, 1, T, logits=False)
    for k in c:
        assert np.array_equal(a[k], c[k]), k


@pytest.mark.parametrize("H", [32, 96, 1056, 4096, 5120, 8160])
def test_one_and_two_rows_match_three(vh, orc, H):
    """Calls of one or two rows stage their activation codes inside the verify
    kernel; a call of three rows uses the separate staging kernel.  The rows'
    logits must agree bit for bit, and with the oracle."""
    V = 3001
    d = synth.uniform_inputs(3, V, H, seed=H + 11, heavy_frac=0.05)
    x = d["hidden"].reshape(3, H).copy()
    x[1, : min(H, 40)] = synth.f16_bits(np.full(min(H, 40), 2.0 ** -24))   # subnormal fp16
    w = dev(d["packed"])
    say(f"one/two/three rows H={H}")
    g3 = run_gpu(vh, x, d["packed"], d["scales"], None, 3, 1, packed_dev=w)
    for M in (1, 2):
        o = oracle_case(orc, x[:M], d["packed"], d["scales"], None, M, 1, V, H)
        g = run_gpu(vh, x[:M], d["packed"], d["scales"], None, M, 1, packed_dev=w)
        parity.check(g, o, M, 1, None)
        assert np.array_equal(g["logits"], g3["logits"][:M])
        assert np.array_equal(g["argmax_ids"], g3["argmax_ids"][:M])
        gl = run_gpu(vh, x[:M], d["packed"], d["scales"], None, M, 1, logits=False, packed_dev=w)
        assert np.array_equal(gl["logits_max"], g3["logits_max"][:M])
        assert np.array_equal(gl["argmax_ids"], g3["argmax_ids"][:M])
    # a verify block of two positions (one draft) takes the same path
    drafts = g3["argmax_ids"][:1].astype(np.int32)
    o = oracle_case(orc, x[:2], d["packed"], d["scales"], drafts, 1, 2, V, H)
    g = run_gpu(vh, x[:2], d["packed"], d["scales"], drafts, 1, 2, packed_dev=w)
    parity.check(g, o, 1, 2, drafts)
    assert g["n_accepted"][0] == 1


@pytest.mark.parametrize("R,T", [(4, 4), (2, 8), (16, 1), (3, 5)])
def test_small_batches(vh, orc, R, T):
    V, H = 5000, 1024
    d = synth.uniform_inputs(R * T, V, H, seed=R * 100 + T)
    o0 = orc.verify(d["hidden"], d["packed"], d["scales"], np.zeros((R, max(T - 1, 0)), np.int32),
                    R, T, V, H, n_threads=NTHREADS)
    am = o0["argmax_ids"].reshape(R, T)
    drafts = am[:, : T - 1].copy()
    for i in range(R):
        if T > 1 and i % 2 == 1:
            drafts[i, i % (T - 1)] = -1
    o = oracle_case(orc, d["hidden"], d["packed"], d["scales"], drafts, R, T, V, H)
    say(f"batch R={R} T={T}")
    g = run_gpu(vh, d["hidden"], d["packed"], d["scales"], drafts, R, T)
    parity.check(g, o, R, T, drafts)


def test_check_weights(vh, orc):
    V, H = 1000, 256
    d = synth.uniform_inputs(1, V, H, seed=4)
    p = d["packed"].copy()
    p[3, 5] = 0x80
    p[999, 127] = 0x88
    p[0, 0] = 0x18
    w = dev(p)
    say("check_weights")
    n = vh.check_weights(w)
    torch.cuda.synchronize()
    assert int(n.item()) == orc.count_bad_nibbles(p, V, H) == 4
    n2 = vh.check_weights(dev(d["packed"]))
    torch.cuda.synchronize()
    assert int(n2.item()) == 0


def test_graph_replay_matches_eager(vh, orc):
    """Verify calls captured in a HIP graph: every replay (with eager work and
    synchronisations in between) equals the eager result of the same call."""
    V, H = 20000, 2048
    calls = []
    for j, T in enumerate((16, 8, 3, 1)):
        d = synth.uniform_inputs(T, V, H, seed=40 + j)
        x = dev(d["hidden"], torch.float16)
        dr = dev(np.arange(max(T - 1, 1), dtype=np.int32))[: max(T - 1, 0)] if T > 1 else None
        calls.append((x, dev(d["packed"]), dev(d["scales"], torch.float16), dr))
    ws = vh.Workspace(vh.workspace_bytes(1, 16, V, H), torch.device("cuda:0"))
    say("graph replay")
    eager = []
    for x, w, s, dr in calls:
        out = vh.verify(x, w, s, dr, logits=True, workspace=ws)
        torch.cuda.synchronize()
        eager.append([o.clone() for o in out])
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    outs = []
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            for x, w, s, dr in calls:
                outs.append(vh.verify(x, w, s, dr, logits=True, workspace=ws))
    torch.cuda.synchronize()
    for rep in range(3):
        for o in outs:
            for t in o:
                t.fill_(-7)
        graph.replay()
        torch.cuda.synchronize()
        for j, (o, e) in enumerate(zip(outs, eager)):
            for a, b in zip(o, e):
                assert torch.equal(a, b), (rep, j)
        # eager work between replays
        x, w, s, dr = calls[rep % len(calls)]
        again = vh.verify(x, w, s, dr, logits=True, workspace=ws)
        torch.cuda.synchronize()
        for a, b in zip(again, eager[rep % len(calls)]):
            assert torch.equal(a, b)

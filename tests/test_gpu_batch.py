"""GPU parity of the batch path (more than 16 rows per call): the HIP path,
through the C ABI, against the CPU oracle on the same seeded inputs."""
import os
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from int4_output_head_amd import synth  # noqa: E402

from . import parity  # noqa: E402

pytestmark = pytest.mark.gpu

NTHREADS = min(16, os.cpu_count() or 1)
HERE = os.path.dirname(os.path.abspath(__file__))


def say(msg):
    print(f"[gpu-batch] {msg}", flush=True)
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


def run_gpu(vh, hidden_bits, packed, scales_bits, drafts, R, T, logits=True, packed_dev=None,
            workspace=None):
    x = dev(hidden_bits, torch.float16)
    w = packed_dev if packed_dev is not None else dev(packed)
    s = dev(scales_bits, torch.float16)
    d = None if T == 1 else dev(np.asarray(drafts, np.int32).reshape(R, T - 1))
    out = vh.verify_batch(x.reshape(R, T, -1), w, s, d, logits=logits, workspace=workspace)
    torch.cuda.synchronize()
    res = dict(logits_max=out[0].cpu().numpy(), argmax_ids=out[1].cpu().numpy(),
               n_accepted=out[2].cpu().numpy())
    if logits:
        res["logits"] = out[3].cpu().numpy()
    return res


def drafts_from(ids, R, T, V, rng):
    """Drafts that copy the given argmax ids with a few planted mismatches."""
    am = np.asarray(ids).reshape(R, T)
    d = am[:, : T - 1].copy()
    for i in range(R):
        if T > 1 and rng.random() < 0.5:
            j = int(rng.integers(0, T - 1))
            d[i, j] = (d[i, j] + 1 + int(rng.integers(0, V - 1))) % V if V > 1 else -1
    return d.astype(np.int32)


# (R, T, V, H): token groups of 16 (17-64 rows) with a partial last group of
# 1, 8, 7 and 5 rows (the last with a ragged 16-row tile and H below one
# 128-channel unit), one 128-row tile, partial tiles, several tiles, a ragged
# last tile, H below one 128-channel step and not a multiple of it, V not a
# multiple of the 128-row vocabulary tile, the 4096-row maximum
CASES = [(17, 1, 1000, 256), (3, 8, 1000, 256), (5, 11, 2500, 640), (3, 7, 129, 32), (4, 8, 3000, 512),
         (64, 2, 2000, 1024), (33, 4, 4097, 640), (64, 4, 1500, 5120), (130, 3, 700, 96),
         (40, 5, 129, 32), (9, 16, 5003, 2080), (256, 16, 300, 128), (4096, 1, 257, 64)]


@pytest.mark.parametrize("R,T,V,H", CASES)
def test_batch_parity(vh, orc, R, T, V, H):
    M = R * T
    d = synth.uniform_inputs(M, V, H, seed=M * 31 + V + H, heavy_frac=0.05)
    o0 = orc.verify(d["hidden"], d["packed"], d["scales"], np.zeros((R, max(T - 1, 0)), np.int32),
                    R, T, V, H, n_threads=NTHREADS)
    drafts = drafts_from(o0["argmax_ids"], R, T, V, np.random.default_rng(M + V))
    o = orc.verify(d["hidden"], d["packed"], d["scales"], drafts, R, T, V, H, want_logits=True,
                   n_threads=NTHREADS)
    say(f"batch parity R={R} T={T} V={V} H={H}")
    g = run_gpu(vh, d["hidden"], d["packed"], d["scales"], drafts, R, T)
    st = parity.check(g, o, R, T, drafts)
    say(f"stats {st}")


@pytest.mark.parametrize("M,V,H", [(40, 1000, 512), (200, 2500, 1024), (17, 4097, 5120)])
def test_batch_int_exact_bitexact(vh, orc, M, V, H):
    """Integer-exact inputs: every summation order gives the same binary32
    bits, so logits, ids (ties included) and acceptance must be bit-exact."""
    d = synth.int_exact_inputs(M, V, H, seed=M + V + H + 1)
    R, T = M, 1
    o = orc.verify(d["hidden"], d["packed"], d["scales"], None, R, T, V, H, want_logits=True,
                   n_threads=NTHREADS)
    say(f"batch int-exact M={M} V={V} H={H}")
    g = run_gpu(vh, d["hidden"], d["packed"], d["scales"], None, R, T)
    assert np.array_equal(g["logits"], o["logits"])
    assert np.array_equal(g["argmax_ids"], o["argmax_ids"])
    assert np.array_equal(g["logits_max"], o["logits_max"])
    assert np.array_equal(g["n_accepted"], o["n_accepted"])


def test_batch_rows_match_single_block_path(vh, orc):
    """The same rows through the batch path (48 rows) and through the
    single-block path (3 calls of 16 rows) give bit-identical results: both
    compute the same exact integer sums and round once."""
    R, T, V, H = 3, 16, 9000, 2048
    d = synth.uniform_inputs(R * T, V, H, seed=77, heavy_frac=0.05)
    drafts = np.full((R, T - 1), -1, np.int32)
    say("batch vs single-block path")
    big = run_gpu(vh, d["hidden"], d["packed"], d["scales"], drafts, R, T)
    x = d["hidden"].reshape(R, T, H)
    for i in range(R):
        one = run_gpu(vh, x[i], d["packed"], d["scales"], drafts[i], 1, T)
        sl = slice(i * T, (i + 1) * T)
        assert np.array_equal(one["logits"], big["logits"][sl])
        assert np.array_equal(one["argmax_ids"], big["argmax_ids"][sl])
        assert np.array_equal(one["logits_max"], big["logits_max"][sl])
        assert one["n_accepted"][0] == big["n_accepted"][i]


def test_token_tiles_bit_identical(vh, orc):
    """The batch path picks a token tile of 32, 64 or 128 rows from the call
    size; the same 24 rows inside calls of 24, 48 and 160 rows (one of each
    tile) give bit-identical logits, maxima and ids, and match the oracle."""
    V, H = 3001, 1280
    d = synth.uniform_inputs(160, V, H, seed=31, heavy_frac=0.05)
    x = d["hidden"].reshape(160, H)
    outs = []
    for M in (24, 48, 160):
        say(f"token tile check M={M}")
        g = run_gpu(vh, np.ascontiguousarray(x[:M]), d["packed"], d["scales"], np.zeros((M, 0), np.int32), M, 1)
        outs.append(g)
    for g in outs[1:]:
        assert np.array_equal(g["logits"][:24], outs[0]["logits"])
        assert np.array_equal(g["argmax_ids"][:24], outs[0]["argmax_ids"])
        assert np.array_equal(g["logits_max"][:24], outs[0]["logits_max"])
    o = orc.verify(np.ascontiguousarray(x[:48]), d["packed"], d["scales"], None, 48, 1, V, H, want_logits=True,
                   n_threads=NTHREADS)
    parity.check(outs[1], o, 48, 1, None)


def test_batch_ties_across_tiles(vh, orc):
    """Copies of the winning row at indices in one vocabulary tile, in other
    tiles and in the last tile: every row's lowest copy must win."""
    M, V, H = 40, 20000, 256
    d = synth.int_exact_inputs(M, V, H, seed=6)
    q = np.clip(d["q"], -3, 3)
    for v in (19999, 12345, 4100, 129, 128, 77):
        q[v] = 7
    x = np.abs(d["hidden"].view(np.float16).astype(np.float64))
    xb = synth.f16_bits(x)
    packed = synth.pack_int4(q)
    R, T = 8, 5
    drafts = np.full((R, T - 1), 77, np.int32)
    drafts[3, 2] = 128
    o = orc.verify(xb, packed, d["scales"], drafts, R, T, V, H, want_logits=True,
                   n_threads=NTHREADS)
    assert np.all(o["argmax_ids"][o["amax"] > 0] == 77)
    say("batch ties across tiles")
    g = run_gpu(vh, xb, packed, d["scales"], drafts, R, T)
    assert np.array_equal(g["argmax_ids"], o["argmax_ids"])
    assert np.array_equal(g["logits"], o["logits"])
    assert np.array_equal(g["n_accepted"], o["n_accepted"])


def test_batch_zero_rows_and_scales(vh, orc):
    """All-zero hidden rows inside a batch, and a batch with zero scales:
    logits are +0, the argmax is 0."""
    R, T, V, H = 20, 2, 700, 256
    d = synth.uniform_inputs(R * T, V, H, seed=8)
    x = d["hidden"].copy()
    x[5] = 0
    x[33] = 0x8000            # -0.0 everywhere
    drafts = np.zeros((R, T - 1), np.int32)
    o = orc.verify(x, d["packed"], d["scales"], drafts, R, T, V, H, want_logits=True,
                   n_threads=NTHREADS)
    say("batch zero rows")
    g = run_gpu(vh, x, d["packed"], d["scales"], drafts, R, T)
    parity.check(g, o, R, T, drafts)
    for r in (5, 33):
        assert np.all(g["logits"][r] == 0) and g["argmax_ids"][r] == 0
    g0 = run_gpu(vh, x, d["packed"], np.zeros(H, np.uint16), drafts, R, T)
    assert np.all(g0["logits"] == 0) and not np.any(np.signbit(g0["logits"]))
    assert np.all(g0["argmax_ids"] == 0) and np.all(g0["n_accepted"] == 1)


def test_batch_workspace_reuse_and_graph_replay(vh, orc):
    """Batch and single-block calls share one workspace, eagerly and in a HIP
    graph replayed several times: the per-row keys are left cleared by every
    call, so every replay equals the eager result."""
    V, H = 6000, 1024
    shapes = [(40, 4), (1, 16), (300, 1), (2, 8)]
    calls = []
    for j, (R, T) in enumerate(shapes):
        d = synth.uniform_inputs(R * T, V, H, seed=50 + j)
        x = dev(d["hidden"], torch.float16).reshape(R, T, H)
        dr = dev(np.arange(R * (T - 1), dtype=np.int32).reshape(R, T - 1) % 97) if T > 1 else None
        calls.append((x, dev(d["packed"]), dev(d["scales"], torch.float16), dr))
    need = max(vh.workspace_bytes(R, T, V, H) for R, T in shapes)
    ws = vh.Workspace(need, torch.device("cuda:0"))
    say("batch workspace reuse and graph replay")
    eager = []
    for x, w, s, dr in calls:
        out = vh.verify_batch(x, w, s, dr, logits=True, workspace=ws)
        torch.cuda.synchronize()
        eager.append([o.clone() for o in out])
    # the same calls again, eagerly: identical
    for (x, w, s, dr), e in zip(calls, eager):
        out = vh.verify_batch(x, w, s, dr, logits=True, workspace=ws)
        torch.cuda.synchronize()
        for a, b in zip(out, e):
            assert torch.equal(a, b)
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    outs = []
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            for x, w, s, dr in calls:
                outs.append(vh.verify_batch(x, w, s, dr, logits=True, workspace=ws))
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
        x, w, s, dr = calls[rep % len(calls)]
        again = vh.verify_batch(x, w, s, dr, logits=True, workspace=ws)
        torch.cuda.synchronize()
        for a, b in zip(again, eager[rep % len(calls)]):
            assert torch.equal(a, b)


def test_batch_config_full_size(vh, orc):
    """64 requests x T=4 over the full-vocabulary head (the launch the
    benchmark times): every row's argmax against the stored oracle argmax
    (ids equal, or a near tie), sampled rows' logits against the oracle, and
    the acceptance counts exactly from the GPU's own ids."""
    import json
    cfg = synth.CONFIGS["batch"]
    path = os.path.join(HERE, "golden", "argmax_batch.json")
    with open(path) as f:
        stored = json.load(f)
    head = synth.make_head(cfg)
    w = dev(head["packed"])
    trial = 0
    x = synth.make_hidden(cfg, trial)
    ref = stored["trials"][str(trial)]
    ids_ref = np.array(ref["argmax"], np.int64)
    gap = np.array(ref["gap"])
    amax = np.array(ref["amax"])
    drafts = synth.finalize_drafts(cfg, synth.draft_plan(cfg, trial), ids_ref)
    say("batch config R=64 T=4 V=151936 H=5120")
    g = run_gpu(vh, x, head["packed"], head["scales"], drafts, cfg.R, cfg.T, logits=True,
                packed_dev=w)
    tol = 2e-3 * amax
    differ = np.nonzero(g["argmax_ids"] != ids_ref)[0]
    assert np.all(gap[differ] < tol[differ]), differ
    assert np.array_equal(g["n_accepted"], parity.accept_from(g["argmax_ids"], drafts, cfg.R,
                                                              cfg.T))
    rows = np.array(sorted({0, 1, 63, 128, 200, 255, *differ.tolist()}))
    lg = orc.logits(np.ascontiguousarray(x.reshape(cfg.M, cfg.H)[rows]), head["packed"],
                    head["scales"], len(rows), cfg.V, cfg.H, n_threads=NTHREADS)
    err = np.max(np.abs(g["logits"][rows].astype(np.float64) - lg), axis=1)
    assert np.all(err <= tol[rows]), err
    assert np.all(np.abs(g["logits_max"] - np.array(
        [g["logits"][r, i] for r, i in enumerate(g["argmax_ids"])])) == 0)
    say(f"ids differ at {differ.tolist()}, max logit error {err.max():.3g}")


@pytest.mark.parametrize("R,T", [(1, 16), (64, 4)])
def test_timed_entry_point(vh, orc, R, T):
    """The instrumented call gives the same results as the plain one, and its
    events bracket the main kernel only: a positive time, shorter than the
    whole call."""
    V, H = 20000, 2048
    d = synth.uniform_inputs(R * T, V, H, seed=90 + R)
    x = dev(d["hidden"], torch.float16).reshape(R, T, H)
    w = dev(d["packed"])
    s = dev(d["scales"], torch.float16)
    dr = dev(np.zeros((R, T - 1), np.int32))
    ws = vh.Workspace(vh.workspace_bytes(R, T, V, H), torch.device("cuda:0"))
    say(f"timed entry point R={R} T={T}")
    plain = vh.verify_batch(x, w, s, dr, logits=True, workspace=ws)
    torch.cuda.synchronize()
    e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    e[0].record()
    timed = vh.verify_batch(x, w, s, dr, logits=True, workspace=ws, events=(e[1], e[2]))
    e[3].record()
    torch.cuda.synchronize()
    for a, b in zip(plain, timed):
        assert torch.equal(a, b)
    t_kernel = e[1].elapsed_time(e[2])
    t_call = e[0].elapsed_time(e[3])
    assert 0 < t_kernel <= t_call
    # either event alone (the other end untimed) is accepted and changes nothing
    for evs in ((e[1], None), (None, e[2])):
        one = vh.verify_batch(x, w, s, dr, logits=True, workspace=ws, events=evs)
        torch.cuda.synchronize()
        for a, b in zip(plain, one):
            assert torch.equal(a, b)

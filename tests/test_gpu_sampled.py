"""GPU parity of sampled verification (verify_lm_head_int4_sampled: top-k
sampling at a temperature, fused into the weight stream) against the oracle
(oracle/sampled.py).  Needs an MI355X and the built library.

Parity rule (from the logit tolerance tol[r] = 2e-3 * max_v |oracle logit|):
  * top-k: the GPU's k ids are distinct, its j-th logit is within tol of the
    oracle's j-th, and the oracle logit at its j-th id is within tol of the
    oracle's j-th (several id lists are correct when logits nearly tie);
  * p_draft: a probability of top-k sampling at temperature tau moves by at
    most a factor exp(2 tol / tau) when every logit moves by at most tol, so
    |p_gpu - p_oracle| <= p_oracle * (exp(2 tol / tau) - 1) + 1e-6 when both
    top-k sets contain the draft, and the draft's logit is within tol of the
    k-th logit whenever only one of them does;
  * n_accepted: exactly the count recomputed from the GPU's own p_draft,
    uniforms and draft probabilities (binary32 product and compare), and the
    oracle's unless the first differing decision is a near tie
    (|u q - p_oracle| within the p_draft bound).

The epilogue's own arithmetic is checked much tighter, separately from the
logit error: the oracle's formulas (top-k probability, log-sum-exp, whole-
vocabulary probability) are evaluated in binary64 on the GPU's own logits
(the greedy path's full logits, which the sampled path reproduces bit for
bit), and the GPU's binary32 results must agree within a bound built from
binary32 rounding: about 1e-5 relative, growing with |logit| / tau (each
exponent argument is rounded once, u |argument|).
"""
import math
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from int4_output_head_amd import synth  # noqa: E402
from oracle import sampled as sm  # noqa: E402

from . import parity  # noqa: E402

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu-sampled] {msg}", flush=True)
    sys.stdout.flush()


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


def make_drafts(lg, R, T, k, seed):
    """Drafts that hit the argmax, other top-k entries, and tokens outside."""
    rng = np.random.default_rng(seed)
    ids, _ = sm.topk_rows(lg, min(k, lg.shape[1]))
    d = np.zeros((R, max(T - 1, 0)), np.int32)
    for i in range(R):
        for t in range(T - 1):
            r = i * T + t
            c = rng.random()
            if c < 0.6:
                d[i, t] = ids[r, 0]
            elif c < 0.85:
                d[i, t] = ids[r, rng.integers(0, ids.shape[1])]
            else:
                d[i, t] = rng.integers(0, lg.shape[1])
    q = rng.uniform(0.3, 1.0, size=d.shape).astype(np.float32)
    q[rng.random(d.shape) < 0.3] = 1.0                      # copied-from-context drafts
    u = rng.random(d.shape).astype(np.float32)
    return d, q, u


def run(vh, inp, d, q, u, R, T, V, H, k, tau):
    T1 = T - 1
    x = dev(inp["hidden"], torch.float16).reshape(R, T, H)
    w = dev(inp["packed"])
    s = dev(inp["scales"], torch.float16)
    out = vh.verify_sampled(x, w, s, dev(d) if T1 else None, dev(q) if T1 else None, dev(u) if T1 else None,
                            top_k=k, temperature=tau, want_lse=True)
    torch.cuda.synchronize()
    names = ("logits_max", "argmax_ids", "topk_ids", "topk_logits", "p_draft", "n_accepted", "lse")
    g = {n: (None if t is None else t.cpu().numpy()) for n, t in zip(names, out)}
    # the GPU's own logits: the greedy call with every logit written
    dd = dev(np.zeros((R, T1), np.int32)) if T1 else None
    g["logits"] = vh.verify_batch(x, w, s, dd, logits=True)[3].cpu().numpy()
    return g


U32 = 2.0 ** -24    # unit roundoff of binary32


def check_own_logits(g, d, R, T, k, tau):
    """The epilogue's arithmetic on the GPU's own logits (binary64 formulas of
    the oracle), with binary32 rounding bounds.  Returns the largest relative
    errors seen."""
    lg = g["logits"].astype(np.float64)
    M, V = lg.shape
    st = dict(own_p_rel=0.0, own_lse_abs=0.0)
    if k > 0:
        # the top-k ids and logits are the GPU's own logits, bit for bit
        for r in range(M):
            assert np.array_equal(g["topk_logits"][r], g["logits"][r, g["topk_ids"][r]]), r
            assert np.array_equal(g["topk_ids"][r], sm.topk_rows(g["logits"][r:r + 1], k)[0][0]), r
    # log-sum-exp over the whole vocabulary
    lse_ref = sm.lse_rows(g["logits"], tau)
    zmax = np.abs(lg).max(axis=1) / tau
    bound_lse = 1e-6 + 8 * U32 * (zmax + np.log(V) + 1)
    err = np.abs(g["lse"].astype(np.float64) - lse_ref)
    assert np.all(err <= bound_lse), (err, bound_lse)
    st["own_lse_abs"] = float(err.max())
    if T == 1:
        return st
    for i in range(R):
        for t in range(T - 1):
            r = i * T + t
            pg = float(g["p_draft"][i, t])
            if k > 0:
                pe = sm.draft_prob(g["topk_ids"][r], g["topk_logits"][r], int(d[i, t]), tau)
                vals = g["topk_logits"][r].astype(np.float64)
                spread = (vals[0] - vals[-1]) / tau
                rel = 1e-5 + 8 * U32 * 2 * spread
            else:
                pe = sm.full_softmax_prob(g["logits"][r], lse_ref[r], int(d[i, t]), tau)
                ld = abs(lg[r, d[i, t]]) / tau if 0 <= d[i, t] < V else 0.0
                rel = 1e-5 + bound_lse[r] + 8 * U32 * ld
            assert abs(pg - pe) <= rel * pe + 1e-35, (i, t, pg, pe, rel)
            if pe > 0:
                st["own_p_rel"] = max(st["own_p_rel"], abs(pg - pe) / pe)
    return st


def check_lse(g, o, lg, tau):
    """|lse_gpu - lse_oracle| <= tol / tau (lse moves by at most max|dlogit| /
    tau) plus the binary32 evaluation."""
    tol = 2e-3 * np.abs(lg.astype(np.float64)).max(axis=1)
    err = np.abs(g["lse"].astype(np.float64) - o["lse"])
    assert np.all(err <= tol / tau + 1e-5 * np.abs(o["lse"]) + 1e-5), (err, tol / tau)
    return float(err.max())


def check(g, o, lg, d, q, u, R, T, k, tau):
    M = R * T
    amax = np.abs(lg.astype(np.float64)).max(axis=1)
    tol = 2e-3 * amax
    stats = dict(topk_ids_differ=0, p_max_rel_err=0.0, accept_near=0)
    # greedy outputs: the usual rule
    gg = dict(logits_max=g["logits_max"], argmax_ids=g["argmax_ids"], n_accepted=np.zeros(R, np.int64))
    oo = dict(o)
    oo["n_accepted"] = np.zeros(R, np.int64)
    parity.check(gg, oo, R, T, np.full((R, max(T - 1, 0)), -1, np.int32))
    assert np.array_equal(g["topk_ids"][:, 0], g["argmax_ids"])
    assert np.array_equal(g["topk_logits"][:, 0], g["logits_max"])
    for r in range(M):
        gi, gv = g["topk_ids"][r], g["topk_logits"][r].astype(np.float64)
        oi, ov = o["topk_ids"][r], o["topk_logits"][r].astype(np.float64)
        assert len(set(gi.tolist())) == k and np.all((gi >= 0) & (gi < lg.shape[1]))
        assert np.all(np.abs(gv - ov) <= tol[r] + 0.0), (r, gv, ov)
        assert np.all(np.abs(lg[r, gi].astype(np.float64) - ov) <= tol[r]), r
        assert np.all(gv[:-1] >= gv[1:])
        if not np.array_equal(gi, oi):
            stats["topk_ids_differ"] += 1
    if T == 1:
        assert np.array_equal(g["n_accepted"], np.zeros(R))
        return stats
    # acceptance from the GPU's own probabilities (binary32 product and compare)
    own = np.zeros(R, np.int64)
    for i in range(R):
        n = 0
        while n < T - 1 and np.float32(u[i, n]) * np.float32(q[i, n]) < g["p_draft"][i, n]:
            n += 1
        own[i] = n
    assert np.array_equal(g["n_accepted"], own)
    near = np.zeros((R, T - 1), bool)
    for i in range(R):
        for t in range(T - 1):
            r = i * T + t
            pg, po = float(g["p_draft"][i, t]), float(o["p_draft"][i, t])
            bound = po * (math.exp(2 * tol[r] / tau) - 1) + 1e-6
            in_g = d[i, t] in g["topk_ids"][r]
            in_o = d[i, t] in o["topk_ids"][r]
            if in_g and in_o:
                assert abs(pg - po) <= bound, (i, t, pg, po, bound)
                if po > 0:
                    stats["p_max_rel_err"] = max(stats["p_max_rel_err"], abs(pg - po) / po)
            elif in_g != in_o:
                # the draft sits at the edge of the top-k: within tol of the k-th logit
                assert abs(float(lg[r, d[i, t]]) - float(o["topk_logits"][r, -1])) <= tol[r], (i, t)
                bound = 1.0
            else:
                assert pg == 0.0 and po == 0.0
            near[i, t] = abs(float(u[i, t]) * float(q[i, t]) - po) <= bound
    for i in range(R):
        if g["n_accepted"][i] != o["n_accepted"][i]:
            first = min(g["n_accepted"][i], o["n_accepted"][i])
            assert near[i, first], f"request {i}: n_accepted {g['n_accepted'][i]} vs {o['n_accepted'][i]}"
            stats["accept_near"] += 1
    return stats


@pytest.mark.parametrize("R,T,V,H,k,tau", [(1, 4, 300, 64, 8, 1.0), (1, 16, 5000, 512, 16, 0.7),
                                           (2, 8, 4097, 256, 5, 1.3), (4, 4, 999, 96, 16, 1.0),
                                           (1, 1, 8192, 5120, 8, 1.0), (3, 5, 2000, 160, 1, 1.0),
                                           (16, 1, 700, 128, 12, 2.0), (1, 16, 5000, 512, 16, 0.3),
                                           (2, 8, 4097, 256, 8, 2.0), (1, 16, 20000, 1024, 16, 1.3),
                                           # more than 16 rows: token groups of 16
                                           (2, 16, 5000, 512, 16, 1.0), (3, 11, 4097, 256, 8, 0.7),
                                           (4, 16, 3000, 128, 16, 1.3), (17, 1, 2000, 96, 5, 2.0),
                                           (5, 12, 20000, 1024, 16, 0.3), (3, 8, 4097, 256, 16, 1.0),
                                           (7, 8, 3000, 128, 8, 0.7),
                                           # more than 64 rows: the batch kernels' logits and
                                           # the per-row selection
                                           (9, 8, 5000, 512, 16, 1.0), (33, 4, 4097, 256, 8, 0.7),
                                           (65, 1, 2000, 96, 5, 2.0), (16, 16, 3000, 128, 16, 0.3),
                                           (100, 3, 600, 64, 12, 1.3), (8, 10, 300, 64, 16, 1.0),
                                           (13, 5, 12, 64, 12, 1.0), (13, 5, 300001, 64, 16, 1.0)])
def test_sampled_parity(vh, oracle_mod, R, T, V, H, k, tau):
    say(f"sampled R={R} T={T} V={V} H={H} k={k} tau={tau}")
    inp = synth.uniform_inputs(R * T, V, H, seed=R * 31 + T + V + H + k)
    lg = oracle_mod.logits(inp["hidden"], inp["packed"], inp["scales"], R * T, V, H)
    d, q, u = make_drafts(lg, R, T, k, seed=V)
    o = sm.verify_sampled(inp["hidden"], inp["packed"], inp["scales"], d, q, u, R, T, V, H, k, tau)
    g = run(vh, inp, d, q, u, R, T, V, H, k, tau)
    st = check(g, o, lg, d, q, u, R, T, k, tau)
    st["lse_max_err"] = check_lse(g, o, lg, tau)
    st.update(check_own_logits(g, d, R, T, k, tau))
    say(f"stats {st}")


def check_full_softmax(g, o, lg, d, q, u, R, T, tau):
    """top_k = 0: p(d) = exp(l_d / tau - lse) moves by at most a factor
    exp(2 tol / tau); acceptance from the GPU's own p exactly, against the
    oracle's up to near ties."""
    amax = np.abs(lg.astype(np.float64)).max(axis=1)
    tol = 2e-3 * amax
    assert g["topk_ids"] is None
    check_lse(g, o, lg, tau)
    near = np.zeros((R, T - 1), bool)
    max_rel = 0.0
    for i in range(R):
        for t in range(T - 1):
            r = i * T + t
            pg, po = float(g["p_draft"][i, t]), float(o["p_draft"][i, t])
            bound = po * (math.exp(2 * tol[r] / tau) - 1) + 1e-6
            assert abs(pg - po) <= bound, (i, t, pg, po)
            if po > 0:
                max_rel = max(max_rel, abs(pg - po) / po)
            near[i, t] = abs(float(u[i, t]) * float(q[i, t]) - po) <= bound
    own = np.zeros(R, np.int64)
    for i in range(R):
        n = 0
        while n < T - 1 and np.float32(u[i, n]) * np.float32(q[i, n]) < g["p_draft"][i, n]:
            n += 1
        own[i] = n
    assert np.array_equal(g["n_accepted"], own)
    for i in range(R):
        if g["n_accepted"][i] != o["n_accepted"][i]:
            assert near[i, min(g["n_accepted"][i], o["n_accepted"][i])]
    return max_rel


@pytest.mark.parametrize("R,T,V,H,tau", [(1, 16, 5000, 512, 1.0), (2, 8, 4097, 256, 0.3),
                                         (4, 4, 999, 96, 2.0), (1, 8, 151936, 5120, 1.0),
                                         (1, 16, 20000, 1024, 0.7), (2, 4, 3000, 256, 1.3),
                                         (2, 16, 5000, 512, 1.0), (4, 16, 3000, 256, 0.7),
                                         (3, 7, 4097, 96, 2.0), (5, 8, 3000, 256, 1.3),
                                         (13, 3, 2000, 96, 0.7),
                                         # more than 64 rows
                                         (9, 8, 5000, 512, 1.0), (40, 4, 4097, 256, 0.7),
                                         (33, 2, 20000, 1024, 2.0)])
def test_full_softmax_parity(vh, oracle_mod, R, T, V, H, tau):
    """Sampling over the whole vocabulary (top_k = 0): the fused online
    log-sum-exp and the draft's probability against the oracle."""
    say(f"full softmax R={R} T={T} V={V} H={H} tau={tau}")
    if V == 151936:
        cfg = synth.CONFIGS["full_t8"]
        head = synth.make_head(cfg)
        inp = dict(hidden=synth.make_hidden(cfg, 0), packed=head["packed"], scales=head["scales"])
    else:
        inp = synth.uniform_inputs(R * T, V, H, seed=V + H)
    lg = oracle_mod.logits(inp["hidden"], inp["packed"], inp["scales"], R * T, V, H, n_threads=16)
    d, q, u = make_drafts(lg, R, T, 8, seed=V)
    d[:, -1] = V + 5                                   # an id outside the vocabulary: p = 0
    lse = sm.lse_rows(lg, tau)
    p, n = sm.sampled_accept(None, None, d, q, u, R, T, tau, logits=lg, lse=lse)
    o = dict(lse=lse, p_draft=p, n_accepted=n)
    g = run(vh, inp, d, q, u, R, T, V, H, 0, tau)
    assert np.all(g["p_draft"][:, -1] == 0.0)
    rel = check_full_softmax(g, o, lg, d, q, u, R, T, tau)
    own = check_own_logits(g, d, R, T, 0, tau)
    say(f"full softmax max relative error of p: {rel:.2e}; on the GPU's own logits {own}")


def test_sampled_full_vocab_two_blocks(vh, oracle_mod):
    """Two T=16 blocks at the full vocabulary (two token groups sharing the
    tile stream), top-16 at tau = 1 and the whole-vocabulary log-sum-exp."""
    cfg = synth.CONFIGS["two_blocks_t16"]
    head = synth.make_head(cfg)
    x = synth.make_hidden(cfg, 0)
    lg = oracle_mod.logits(x, head["packed"], head["scales"], cfg.M, cfg.V, cfg.H, n_threads=16)
    inp = dict(hidden=x, packed=head["packed"], scales=head["scales"])
    d, q, u = make_drafts(lg, cfg.R, cfg.T, 16, seed=4)
    ids, vals = sm.topk_rows(lg, 16)
    idx, mx, gap, amax = oracle_mod.argmax_rows(lg)
    p, n = sm.sampled_accept(ids, vals, d, q, u, cfg.R, cfg.T, 1.0)
    o = dict(logits=lg, logits_max=mx, argmax_ids=idx, gap=gap, amax=amax, topk_ids=ids,
             topk_logits=vals, p_draft=p, n_accepted=n, lse=sm.lse_rows(lg, 1.0))
    g = run(vh, inp, d, q, u, cfg.R, cfg.T, cfg.V, cfg.H, 16, 1.0)
    st = check(g, o, lg, d, q, u, cfg.R, cfg.T, 16, 1.0)
    st["lse_max_err"] = check_lse(g, o, lg, 1.0)
    st.update(check_own_logits(g, d, cfg.R, cfg.T, 16, 1.0))
    say(f"full-vocab 2 x T=16 stats {st}")


def test_sampled_full_vocab_t16(vh, oracle_mod):
    """The headline shape: V=151936, H=5120, T=16, top-16 at tau = 1."""
    cfg = synth.CONFIGS["full_t16"]
    head = synth.make_head(cfg)
    x = synth.make_hidden(cfg, 0)
    lg = oracle_mod.logits(x, head["packed"], head["scales"], cfg.M, cfg.V, cfg.H, n_threads=16)
    inp = dict(hidden=x, packed=head["packed"], scales=head["scales"])
    d, q, u = make_drafts(lg, 1, 16, 16, seed=1)
    ids, vals = sm.topk_rows(lg, 16)
    idx, mx, gap, amax = oracle_mod.argmax_rows(lg)
    p, n = sm.sampled_accept(ids, vals, d, q, u, 1, 16, 1.0)
    o = dict(logits=lg, logits_max=mx, argmax_ids=idx, gap=gap, amax=amax, topk_ids=ids,
             topk_logits=vals, p_draft=p, n_accepted=n)
    g = run(vh, inp, d, q, u, 1, 16, cfg.V, cfg.H, 16, 1.0)
    st = check(g, o, lg, d, q, u, 1, 16, 16, 1.0)
    st.update(check_own_logits(g, d, 1, 16, 16, 1.0))
    say(f"full-vocab T=16 stats {st}")


@pytest.mark.parametrize("R,T", [(2, 8), (3, 16), (9, 8), (20, 4)])
def test_sampled_int_exact_bitexact(vh, oracle_mod, R, T):
    """Integer-exact inputs: the top-k ids (ties broken by the lowest row
    across tiles and workgroups) and logits equal the oracle's bit for bit
    (one block of 16 rows, three token groups, and beyond 64 rows the
    per-row selection over the batch kernels' logits)."""
    V, H, k = 3000, 512, 16
    inp = synth.int_exact_inputs(R * T, V, H, seed=12)
    lg = oracle_mod.logits(inp["hidden"], inp["packed"], inp["scales"], R * T, V, H)
    d, q, u = make_drafts(lg, R, T, k, seed=2)
    o = sm.verify_sampled(inp["hidden"], inp["packed"], inp["scales"], d, q, u, R, T, V, H, k, 1.0)
    g = run(vh, inp, d, q, u, R, T, V, H, k, 1.0)
    assert np.array_equal(g["topk_ids"], o["topk_ids"])
    assert np.array_equal(g["topk_logits"], o["topk_logits"])
    assert np.allclose(g["p_draft"], o["p_draft"], rtol=1e-5, atol=1e-7)
    check(g, o, lg, d, q, u, R, T, k, 1.0)


@pytest.mark.parametrize("k,H", [(16, 512), (8, 5120), (16, 7296)])
def test_sampled_monotone_logits(vh, oracle_mod, k, H):
    """Head rows reordered so that token 0's logits rise along the vocabulary
    (every tile's keys beat the list: the candidate buffer fills and is
    sorted into the list tile after tile), token 1's (the negated hidden
    state, exact) fall (no candidates after the first tile), token 2 random.
    H = 7296 takes the direct-insertion path (no LDS room for the buffer)."""
    R, T, V = 1, 3, 6000
    say(f"monotone logits k={k} H={H}")
    inp = synth.uniform_inputs(R * T, V, H, seed=k + H)
    x = inp["hidden"].reshape(R * T, H).copy()
    x[1] = x[0] ^ np.uint16(0x8000)                    # exact negation of token 0
    lg0 = oracle_mod.logits(x[:1], inp["packed"], inp["scales"], 1, V, H)
    order = np.argsort(lg0[0], kind="stable")          # ascending logits of token 0
    packed = inp["packed"].reshape(V, H // 2)[order].copy()
    inp = dict(hidden=x, packed=packed, scales=inp["scales"])
    lg = oracle_mod.logits(x, packed, inp["scales"], R * T, V, H)
    assert np.all(np.diff(lg[0].astype(np.float64)) >= 0)
    d, q, u = make_drafts(lg, R, T, k, seed=3)
    o = sm.verify_sampled(x, packed, inp["scales"], d, q, u, R, T, V, H, k, 1.0)
    g = run(vh, inp, d, q, u, R, T, V, H, k, 1.0)
    st = check(g, o, lg, d, q, u, R, T, k, 1.0)
    st.update(check_own_logits(g, d, R, T, k, 1.0))
    say(f"monotone stats {st}")


def test_k1_is_greedy_acceptance(vh):
    """top_k = 1: the argmax has probability 1, every other token 0, so with
    draft probabilities 1 and uniforms below 1 the sampled count equals the
    greedy count of verify_lm_head_int4."""
    R, T, V, H = 1, 16, 20000, 1024
    inp = synth.uniform_inputs(T, V, H, seed=77)
    x = dev(inp["hidden"], torch.float16)
    w = dev(inp["packed"])
    s = dev(inp["scales"], torch.float16)
    _, ids, _ = vh.verify(x, w, s, dev(np.zeros(T - 1, np.int32)))
    d = ids[: T - 1].clone()
    d[9] = (d[9] + 1) % V
    q = torch.ones(T - 1, dtype=torch.float32, device="cuda")
    u = torch.full((T - 1,), 0.999, dtype=torch.float32, device="cuda")
    lmax_g, ids_g, n_g = vh.verify(x, w, s, d)
    out = vh.verify_sampled(x.reshape(1, T, H), w, s, d, q, u, top_k=1, temperature=1.0)
    torch.cuda.synchronize()
    assert int(out[5].item()) == int(n_g.item()) == 9
    assert torch.equal(out[0], lmax_g) and torch.equal(out[1], ids_g)
    assert torch.all(out[4][0, :9] == 1.0) and float(out[4][0, 9]) == 0.0


@pytest.mark.parametrize("R,T", [(1, 8), (3, 12), (20, 4)])
def test_sampled_then_greedy_workspace_reuse(vh, R, T):
    """Sampled and greedy calls alternate on one workspace; each call leaves
    it ready for the next (results equal fresh calls), with one block, with
    token groups and with the batch path."""
    V, H = 6000, 256
    inp = synth.uniform_inputs(R * T, V, H, seed=5 + R)
    x = dev(inp["hidden"], torch.float16).reshape(R, T, H)
    w = dev(inp["packed"])
    s = dev(inp["scales"], torch.float16)
    d = dev((np.arange(R * (T - 1), dtype=np.int32) % V).reshape(R, T - 1))
    q = torch.ones((R, T - 1), dtype=torch.float32, device="cuda")
    u = torch.rand((R, T - 1), dtype=torch.float32, device="cuda")
    ws = vh.Workspace(vh.sampled_workspace_bytes(R, T, V, H), x.device)
    a1 = vh.verify_sampled(x, w, s, d, q, u, top_k=16, workspace=ws)
    b1 = vh.verify_batch(x, w, s, d, workspace=ws)
    a2 = vh.verify_sampled(x, w, s, d, q, u, top_k=16, workspace=ws)
    b2 = vh.verify_batch(x, w, s, d, workspace=ws)
    torch.cuda.synchronize()
    for p1, p2 in zip(a1, a2):
        assert (p1 is None and p2 is None) or torch.equal(p1, p2)
    for p1, p2 in zip(b1, b2):
        assert torch.equal(p1, p2)


def test_batch_sampled_crowded_slice(vh, oracle_mod):
    """More than 64 rows, integer-exact logits built so that each row's
    largest values tie at rows v = c0, c0 + 512, ... (one row in every fourth
    vocabulary tile of 128) above a crowd of tied second-largest values (every
    third row): the selection's threshold and candidates rest on tied keys and
    the order falls to the lowest rows.  Top-k ids and logits equal the
    oracle's bit for bit, and p(d) the oracle's formula on them."""
    R, T, V, H, k = 33, 2, 10000, 64, 16
    M = R * T
    say(f"crowded slice R={R} T={T} V={V} H={H} k={k}")
    inp = synth.int_exact_inputs(M, V, H, seed=21)
    q = inp["q"].copy()
    rng = np.random.default_rng(5)
    rows = np.arange(V)
    for c in range(H):
        q[:, c] = rng.integers(-7, 6, size=V)             # below the two top values
        q[rows % 3 == c % 3, c] = 6                        # a crowd of second-largest values
        q[rows % 512 == (7 * c) % 512, c] = 7              # the largest: one slice of 512
    x = np.zeros((M, H))
    x[np.arange(M), np.arange(M) % H] = 1.0                # row m reads channel m % H
    inp = dict(hidden=synth.f16_bits(x), packed=synth.pack_int4(q), scales=inp["scales"])
    lg = oracle_mod.logits(inp["hidden"], inp["packed"], inp["scales"], M, V, H)
    d, qd, u = make_drafts(lg, R, T, k, seed=6)
    o = sm.verify_sampled(inp["hidden"], inp["packed"], inp["scales"], d, qd, u, R, T, V, H, k, 1.0)
    g = run(vh, inp, d, qd, u, R, T, V, H, k, 1.0)
    assert np.array_equal(g["topk_ids"], o["topk_ids"])
    assert np.array_equal(g["topk_logits"], o["topk_logits"])
    for m in range(M):                                 # the 16 best are the slice's first 16 rows
        c0 = (7 * (m % H)) % 512
        assert np.array_equal(g["topk_ids"][m], c0 + 512 * np.arange(16)), m
    assert np.allclose(g["p_draft"], o["p_draft"], rtol=1e-5, atol=1e-7)
    check(g, o, lg, d, qd, u, R, T, k, 1.0)
    check_own_logits(g, d, R, T, k, 1.0)


def test_batch_sampled_full_vocab(vh, oracle_mod):
    """More than 64 rows at the full vocabulary (V = 151936, H = 5120: 1187
    tile keys per row): 9 requests x T = 8, top-16 at tau = 0.7 with the
    log-sum-exp, against the oracle and on the GPU's own logits."""
    R, T, k, tau = 9, 8, 16, 0.7
    cfg = synth.CONFIGS["full_t16"]
    head = synth.make_head(cfg)
    x = np.concatenate([synth.make_hidden(cfg, s) for s in range(5)])[: R * T]
    lg = oracle_mod.logits(x, head["packed"], head["scales"], R * T, cfg.V, cfg.H, n_threads=16)
    inp = dict(hidden=x, packed=head["packed"], scales=head["scales"])
    d, q, u = make_drafts(lg, R, T, k, seed=9)
    ids, vals = sm.topk_rows(lg, k)
    idx, mx, gap, amax = oracle_mod.argmax_rows(lg)
    p, n = sm.sampled_accept(ids, vals, d, q, u, R, T, tau)
    o = dict(logits=lg, logits_max=mx, argmax_ids=idx, gap=gap, amax=amax, topk_ids=ids,
             topk_logits=vals, p_draft=p, n_accepted=n, lse=sm.lse_rows(lg, tau))
    g = run(vh, inp, d, q, u, R, T, cfg.V, cfg.H, k, tau)
    st = check(g, o, lg, d, q, u, R, T, k, tau)
    st["lse_max_err"] = check_lse(g, o, lg, tau)
    st.update(check_own_logits(g, d, R, T, k, tau))
    say(f"full-vocab 9 x T=8 (batch path) stats {st}")


@pytest.mark.parametrize("R,T,k", [(9, 8, 16), (33, 2, 8)])
def test_batch_sampled_without_lse(vh, R, T, k):
    """More than 64 rows without the log-sum-exp (the selection's top-k-only
    instance): top-k ids and logits, p(d) and the accepted counts equal the
    call that also returns the log-sum-exp, bit for bit."""
    V, H = 7000, 256
    inp = synth.uniform_inputs(R * T, V, H, seed=R + T + k)
    x = dev(inp["hidden"], torch.float16).reshape(R, T, H)
    w = dev(inp["packed"])
    s = dev(inp["scales"], torch.float16)
    rng = np.random.default_rng(k)
    d = dev(rng.integers(0, V, (R, T - 1), dtype=np.int32))
    q = dev(rng.uniform(0.3, 1.0, (R, T - 1)).astype(np.float32))
    u = dev(rng.random((R, T - 1)).astype(np.float32))
    a1 = vh.verify_sampled(x, w, s, d, q, u, top_k=k, temperature=0.8)
    a2 = vh.verify_sampled(x, w, s, d, q, u, top_k=k, temperature=0.8, want_lse=True)
    torch.cuda.synchronize()
    assert a1[6] is None and a2[6] is not None
    for t1, t2 in zip(a1[:6], a2[:6]):
        assert torch.equal(t1, t2)

"""Pins of the sampled-verification oracle (oracle/sampled.py): top-k against
a full sort and the greedy oracle, probabilities against closed forms, the
acceptance rule on hand cases, and its limits (k = 1 / low temperature turn
it into the greedy rule for sure drafts)."""
import math

import numpy as np
import pytest

from int4_output_head_amd import synth
from oracle import sampled as sm


def test_topk_matches_full_sort_and_greedy(oracle_mod):
    M, V, H = 5, 700, 64
    inp = synth.uniform_inputs(M, V, H, seed=3)
    lg = oracle_mod.logits(inp["hidden"], inp["packed"], inp["scales"], M, V, H)
    ids, vals = sm.topk_rows(lg, 16)
    for r in range(M):
        srt = sorted(range(V), key=lambda v: (-float(lg[r, v]), v))[:16]
        assert ids[r].tolist() == srt
        assert np.array_equal(vals[r], lg[r, srt])
    idx, mx, _, _ = oracle_mod.argmax_rows(lg)
    assert np.array_equal(ids[:, 0], idx) and np.array_equal(vals[:, 0], mx)


def test_topk_ties_prefer_lower_rows(oracle_mod):
    d = synth.int_exact_inputs(4, 400, 32, seed=2)    # integer logits: many exact ties
    lg = oracle_mod.logits(d["hidden"], d["packed"], d["scales"], 4, 400, 32)
    ids, vals = sm.topk_rows(lg, 16)
    for r in range(4):
        for j in range(15):
            assert vals[r, j] > vals[r, j + 1] or (vals[r, j] == vals[r, j + 1] and ids[r, j] < ids[r, j + 1])
    assert any(vals[r, j] == vals[r, j + 1] for r in range(4) for j in range(15))


def test_draft_prob_closed_forms():
    ids = np.array([7, 3, 9], np.int32)
    vals = np.array([2.0, 1.0, 0.0], np.float32)
    z = 1 + math.exp(-1) + math.exp(-2)
    assert sm.draft_prob(ids, vals, 7, 1.0) == pytest.approx(1 / z, rel=1e-15)
    assert sm.draft_prob(ids, vals, 9, 1.0) == pytest.approx(math.exp(-2) / z, rel=1e-15)
    assert sm.draft_prob(ids, vals, 4, 1.0) == 0.0                  # outside the top-k
    z2 = 1 + math.exp(-2) + math.exp(-4)
    assert sm.draft_prob(ids, vals, 3, 0.5) == pytest.approx(math.exp(-2) / z2, rel=1e-15)
    # equal logits: uniform over the k
    assert sm.draft_prob(ids, np.zeros(3, np.float32), 3, 0.7) == pytest.approx(1 / 3, rel=1e-15)
    # k = 1: the argmax has probability 1
    assert sm.draft_prob(ids[:1], vals[:1], 7, 3.0) == 1.0


def test_acceptance_rule_hand_cases():
    R, T = 2, 4
    top_ids = np.array([[5, 6], [1, 2], [3, 4], [0, 9], [5, 6], [1, 2], [3, 4], [0, 9]], np.int32)
    top_vals = np.zeros((8, 2), np.float32)          # p = 1/2 for either of the two
    drafts = np.array([[5, 2, 4], [6, 1, 8]], np.int32)
    q = np.ones((R, T - 1))
    u = np.array([[0.1, 0.49, 0.51], [0.3, 0.2, 0.0]])
    p, n = sm.sampled_accept(top_ids, top_vals, drafts, q, u, R, T, 1.0)
    assert np.allclose(p, [[0.5, 0.5, 0.5], [0.5, 0.5, 0.0]])
    assert n.tolist() == [2, 2]        # request 0 stops at u=0.51; request 1 at token 8 (p=0)
    # a drafter that was sure of a token (q = 1) versus one that was unsure (q = 0.5)
    q2 = np.array([[1.0, 1.0, 0.5], [1.0, 1.0, 1.0]])
    _, n2 = sm.sampled_accept(top_ids, top_vals, drafts, q2, u, R, T, 1.0)
    assert n2.tolist() == [3, 2]       # 0.51 * 0.5 < 0.5
    _, n1 = sm.sampled_accept(top_ids, top_vals, drafts, q, u, R, 1, 1.0)
    assert n1.tolist() == [0, 0]


def test_greedy_limit(oracle_mod):
    """k = 1 (or a tiny temperature with a clear maximum): drafts equal to the
    argmax are always accepted and others always rejected, which is the
    greedy rule of the verify oracle."""
    R, T, V, H = 1, 8, 500, 96
    inp = synth.uniform_inputs(T, V, H, seed=11)
    g = oracle_mod.verify(inp["hidden"], inp["packed"], inp["scales"], np.zeros(T - 1, np.int32),
                          R, T, V, H)
    d = np.asarray(g["argmax_ids"][: T - 1], np.int32).copy()
    d[4] = (d[4] + 1) % V
    u = np.random.default_rng(0).random((R, T - 1)) * 0.999
    q = np.ones((R, T - 1))
    for k, tau in ((1, 1.0), (16, 1e-4)):
        o = sm.verify_sampled(inp["hidden"], inp["packed"], inp["scales"], d, q, u, R, T, V, H, k, tau)
        assert int(o["n_accepted"][0]) == 4
        gg = oracle_mod.verify(inp["hidden"], inp["packed"], inp["scales"], d, R, T, V, H)
        assert int(gg["n_accepted"][0]) == 4


def test_lse_and_full_softmax_closed_forms():
    lg = np.array([[2.0, 1.0, 0.0, -1.0]], np.float32)
    for tau in (1.0, 0.5, 3.0):
        lse = sm.lse_rows(lg, tau)[0]
        want = math.log(sum(math.exp(v / tau) for v in (2.0, 1.0, 0.0, -1.0)))
        assert lse == pytest.approx(want, rel=1e-15)
        assert sm.full_softmax_prob(lg[0], lse, 1, tau) == pytest.approx(
            math.exp(1.0 / tau) / sum(math.exp(v / tau) for v in (2.0, 1.0, 0.0, -1.0)), rel=1e-14)
    assert sm.full_softmax_prob(lg[0], 0.0, 4, 1.0) == 0.0 and sm.full_softmax_prob(lg[0], 0.0, -1, 1.0) == 0.0
    # large logits: the factored maximum keeps it finite
    big = np.array([[1000.0, 999.0]], np.float32)
    assert sm.lse_rows(big, 1.0)[0] == pytest.approx(1000.0 + math.log(1 + math.exp(-1)), rel=1e-15)
    # probabilities over the whole vocabulary sum to one
    rng = np.random.default_rng(0)
    row = rng.normal(0, 7, size=500).astype(np.float32)
    lse = sm.lse_rows(row[None, :], 0.8)[0]
    assert sum(sm.full_softmax_prob(row, lse, v, 0.8) for v in range(500)) == pytest.approx(1.0, abs=1e-12)


def test_full_softmax_acceptance_vs_topk(oracle_mod):
    """k = 0 (the whole vocabulary) gives each draft a probability no larger
    than top-k sampling does when the draft is among the top k."""
    R, T, V, H = 1, 8, 400, 64
    inp = synth.uniform_inputs(T, V, H, seed=4)
    g = oracle_mod.verify(inp["hidden"], inp["packed"], inp["scales"], np.zeros(T - 1, np.int32), R, T, V, H)
    d = np.asarray(g["argmax_ids"][: T - 1], np.int32)
    q = np.ones((R, T - 1))
    u = np.full((R, T - 1), 0.3)
    full = sm.verify_sampled(inp["hidden"], inp["packed"], inp["scales"], d, q, u, R, T, V, H, 0, 1.0)
    top = sm.verify_sampled(inp["hidden"], inp["packed"], inp["scales"], d, q, u, R, T, V, H, 16, 1.0)
    assert np.all(full["p_draft"] <= top["p_draft"] + 1e-15)
    assert full["topk_ids"] is None and full["lse"].shape == (T,)
    assert np.allclose(full["lse"], top["lse"])

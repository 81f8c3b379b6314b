"""CPU oracle of sampled (non-greedy) verification through the int4 head.

TEST INFRASTRUCTURE ONLY: imported by the test suite and the benchmark's
CPU-baseline leg, never by the GPU library or its binding.

Source: "HyperQwen: 1,000 tok/s on a Single RTX 3090 Through Aggressive
Recurrent-State Speculation", Technical Insight (lm_head paragraph): the
int4 head is good enough because top-k sampling needs only the relative
ordering of the logits.  The verify step of "Qwen3.8-27B on a Single RTX
3090: How Calibrated Quantization and Speculative Decoding Hit 1,000 tok/s",
Technical Insight (split-KV verify listing), keeps the accepted prefix of
the drafted block.  The pages give no sampled acceptance rule; the readings
used (standard speculative sampling restricted to a top-k target):

  * the target distribution of a position is top-k sampling at temperature
    tau: the k largest logits (ties: lower vocabulary row first), softmax of
    logit / tau over those k, probability 0 outside them;
  * drafted token d_t, proposed with probability q_t by the drafter (1 for a
    token copied from the context), is accepted when u_t * q_t < p_t(d_t),
    with u_t uniform in [0, 1) supplied by the caller; the accepted count is
    the number of leading accepted drafts (the first rejection stops);
  * with k = 0 the target distribution is plain sampling at temperature
    tau over the whole vocabulary: p(d) = exp(logit_d / tau - lse), where
    lse = log sum_v exp(logit_v / tau) (ids outside the vocabulary: p = 0);
    lse is reported for every row in both modes;
  * the replacement or bonus token is drawn by the caller from the top-k
    outputs (it needs the drafter's full distribution for the residual).

Arithmetic: the logits are the verify oracle's (binary32, pinned); top-k
selection is an ordering of those values; the probabilities are evaluated in
binary64 from them.
"""
from __future__ import annotations

import numpy as np

from . import oracle


def topk_rows(logits: np.ndarray, k: int):
    """Per row the k best (value desc, then lower index) ids and values."""
    lg = np.asarray(logits, np.float32)
    M, V = lg.shape
    if not 1 <= k <= V:
        raise ValueError("need 1 <= k <= V")
    ids = np.empty((M, k), np.int32)
    vals = np.empty((M, k), np.float32)
    cols = np.arange(V)
    for r in range(M):
        # lexicographic: larger value first, then smaller index (-0.0 == +0.0)
        order = np.lexsort((cols, -lg[r].astype(np.float64)))[:k]
        ids[r] = order
        vals[r] = lg[r, order]
    return ids, vals


def draft_prob(top_ids, top_vals, d: int, tau: float) -> float:
    """p(d) under top-k sampling at temperature tau (binary64)."""
    v = np.asarray(top_vals, np.float64)
    w = np.exp((v - v[0]) / tau)
    hit = np.nonzero(np.asarray(top_ids) == d)[0]
    return float(w[hit[0]] / w.sum()) if hit.size else 0.0


def lse_rows(logits, tau: float) -> np.ndarray:
    """log sum_v exp(logit / tau) per row, binary64, evaluated with the
    row maximum factored out."""
    z = np.asarray(logits, np.float64) / tau
    m = z.max(axis=1)
    return m + np.log(np.exp(z - m[:, None]).sum(axis=1))


def full_softmax_prob(logit_row, lse: float, d: int, tau: float) -> float:
    """p(d) under sampling over the whole vocabulary at temperature tau."""
    if not 0 <= d < len(logit_row):
        return 0.0
    return float(np.exp(np.float64(logit_row[d]) / tau - lse))


def sampled_accept(top_ids, top_vals, draft_ids, draft_probs, uniforms, R: int, T: int, tau: float,
                   logits=None, lse=None):
    """p_draft [R, T-1] and the accepted count per request: top-k sampling,
    or with logits and lse given, sampling over the whole vocabulary."""
    n = np.zeros(R, np.int32)
    p = np.zeros((R, max(T - 1, 0)), np.float64)
    if T == 1:
        return p, n
    d = np.asarray(draft_ids, np.int64).reshape(R, T - 1)
    q = np.asarray(draft_probs, np.float64).reshape(R, T - 1)
    u = np.asarray(uniforms, np.float64).reshape(R, T - 1)
    for i in range(R):
        for t in range(T - 1):
            r = i * T + t
            if logits is None:
                p[i, t] = draft_prob(top_ids[r], top_vals[r], int(d[i, t]), tau)
            else:
                p[i, t] = full_softmax_prob(logits[r], lse[r], int(d[i, t]), tau)
        k = 0
        while k < T - 1 and u[i, k] * q[i, k] < p[i, k]:
            k += 1
        n[i] = k
    return p, n


def verify_sampled(hidden_bits, packed, scales_bits, draft_ids, draft_probs, uniforms, R: int, T: int,
                   V: int, H: int, k: int, tau: float, n_threads: int = 0) -> dict:
    if not tau > 0:
        raise ValueError("temperature must be > 0")
    lg = oracle.logits(hidden_bits, packed, scales_bits, R * T, V, H, n_threads=n_threads)
    idx, mx, gap, amax = oracle.argmax_rows(lg)
    lse = lse_rows(lg, tau)
    if k > 0:
        ids, vals = topk_rows(lg, k)
        p, n = sampled_accept(ids, vals, draft_ids, draft_probs, uniforms, R, T, tau)
    else:
        ids = vals = None
        p, n = sampled_accept(None, None, draft_ids, draft_probs, uniforms, R, T, tau, logits=lg, lse=lse)
    return dict(logits=lg, logits_max=mx, argmax_ids=idx, gap=gap, amax=amax, topk_ids=ids,
                topk_logits=vals, lse=lse, p_draft=p, n_accepted=n)

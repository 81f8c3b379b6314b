"""CPU oracle of the context-copy (prompt lookup) drafter that fills verify
positions 7-14 from the request's own prompt.

TEST INFRASTRUCTURE ONLY: imported by the test suite and the benchmark's
CPU-baseline leg, never by the GPU library or its binding.

Sources: "Qwen3.8-27B on a Single RTX 3090: How Calibrated Quantization and
Speculative Decoding Hit 1,000 tok/s", Technical Insight (the
draft-from-context optimisation: positions 7-14 of the verify block are
copied from the prompt instead of being drafted); "HyperQwen: 1,000 tok/s on
a Single RTX 3090 Through Aggressive Recurrent-State Speculation", Technical
Insight (positions 7-14 draft from the request's own context); "HyperQwen on
one RTX 3090: a first-time developer's guide to the 381-token claim", "What
actually became faster?" (a lookup proposes further tokens straight from
the context when the answer starts copying it); the HyperQwen README names
it the lookup drafter.  The pages give no algorithm; the reading used here
(plain prompt lookup):

  * key = the last n_max tokens of the sequence so far (the committed
    tokens followed by the 7 model-drafted ones);
  * for every end position e of the prompt with 1 <= e <= L-1 (at least one
    prompt token follows), the match length l(e) is the number of key tokens
    that match the prompt going backwards from e:
    prompt[e-1-i] == key[n_max-1-i] for i < l(e), l(e) <= min(n_max, e);
  * the match is the largest l(e) >= n_min, and among equal lengths the
    latest e (the most recent occurrence);
  * the proposal is prompt[e : e + min(n_out, L - e)] (n_out = 8 for
    positions 7-14); with no match of length >= n_min nothing is proposed.
"""
from __future__ import annotations

import numpy as np


def match_lengths(prompt, key) -> np.ndarray:
    """l(e) for e = 0 .. L-1 (l(0) = 0; position e compares prompt[e-1-i]
    with key[-1-i])."""
    p = np.asarray(prompt, np.int64)
    k = np.asarray(key, np.int64)
    L, n = p.size, k.size
    ell = np.zeros(L, np.int64)
    alive = np.ones(L, bool)
    alive[0] = False
    for i in range(n):
        e = np.arange(L)
        idx = e - 1 - i
        ok = alive & (idx >= 0)
        ok[ok] = p[idx[ok]] == k[n - 1 - i]
        ell[ok] += 1
        alive = ok
    return ell


def propose(prompt, key, n_min: int, n_out: int) -> dict:
    """Returns tokens (int32 [count]), count, match_end (-1 if none) and
    match_len (0 if none)."""
    p = np.asarray(prompt, np.int64)
    L = p.size
    n_max = len(key)
    if not (1 <= n_min <= n_max) or n_out < 1:
        raise ValueError("need 1 <= n_min <= n_max and n_out >= 1")
    if L < 2:
        return dict(tokens=np.zeros(0, np.int32), count=0, match_end=-1, match_len=0)
    cand = match_lengths(p, key)     # e = 0 .. L-1: every e <= L-1 has a following token
    best = int(cand.max())
    if best < n_min:
        return dict(tokens=np.zeros(0, np.int32), count=0, match_end=-1, match_len=0)
    e = int(np.nonzero(cand == best)[0][-1])
    cnt = min(n_out, L - e)
    return dict(tokens=p[e:e + cnt].astype(np.int32), count=cnt, match_end=e, match_len=best)

"""Parity rule between the GPU path and the oracle (test helper, not a test).

Per row r, tol[r] = 2e-3 * max_v |oracle logit[r, v]| (exact agreement is
required when that maximum is 0):
  * logits (when compared): max_v |gpu - oracle| <= tol[r];
  * logits_max: |gpu - oracle| <= tol[r];
  * argmax: equal to the oracle's, or a near tie: the oracle's logit at the
    GPU's id is within tol[r] of the oracle's maximum (counted);
  * n_accepted: exactly the accepted prefix recomputed from the GPU's own
    argmax ids and the drafts; equal to the oracle's unless the first
    differing position is a near-tie row (counted).
"""
from __future__ import annotations

import numpy as np

TOL_REL = 2e-3


def accept_from(ids, drafts, R, T):
    ids = np.asarray(ids).reshape(R, T)
    out = np.zeros(R, np.int64)
    if T == 1:
        return out
    d = np.asarray(drafts).reshape(R, T - 1)
    for i in range(R):
        n = 0
        while n < T - 1 and ids[i, n] == d[i, n]:
            n += 1
        out[i] = n
    return out


def check(gpu: dict, orc: dict, R: int, T: int, drafts=None, orc_logit_at=None,
          tol_rel: float = TOL_REL) -> dict:
    """gpu: logits_max, argmax_ids, n_accepted (+ optional logits) as numpy.
    orc: oracle.verify() output (with 'logits' when full logits are compared).
    orc_logit_at(r, v) returns the oracle logit of one entry when the full
    oracle logits are not at hand.  Raises AssertionError on a violation and
    returns counts."""
    M = R * T
    amax = np.asarray(orc["amax"], np.float64)
    tol = tol_rel * amax
    stats = dict(rows=M, near_tie_rows=int(np.sum(orc["gap"] < tol)), ids_differ=0,
                 accept_divergence=0, max_abs_err=0.0, max_rel_err=0.0)

    if "logits" in gpu and gpu["logits"] is not None and "logits" in orc:
        g = np.asarray(gpu["logits"], np.float64)
        o = np.asarray(orc["logits"], np.float64)
        err = np.max(np.abs(g - o), axis=1)
        for r in range(M):
            if amax[r] == 0:
                assert err[r] == 0, f"row {r}: oracle logits are all zero, GPU differs by {err[r]}"
            else:
                assert err[r] <= tol[r], f"row {r}: logit error {err[r]} > tol {tol[r]}"
        stats["max_abs_err"] = float(err.max())
        nz = amax > 0
        if nz.any():
            stats["max_rel_err"] = float(np.max(err[nz] / amax[nz]))

    gm = np.asarray(gpu["logits_max"], np.float64)
    om = np.asarray(orc["logits_max"], np.float64)
    for r in range(M):
        assert abs(gm[r] - om[r]) <= tol[r], f"row {r}: logits_max {gm[r]} vs {om[r]} (tol {tol[r]})"

    gi = np.asarray(gpu["argmax_ids"], np.int64)
    oi = np.asarray(orc["argmax_ids"], np.int64)
    near = np.zeros(M, bool)
    for r in range(M):
        if gi[r] == oi[r]:
            continue
        if orc_logit_at is not None:
            ov = orc_logit_at(r, int(gi[r]))
        else:
            ov = float(orc["logits"][r, gi[r]])
        assert 0 <= gi[r] and ov >= om[r] - tol[r], (
            f"row {r}: GPU id {gi[r]} (oracle logit {ov}) vs oracle id {oi[r]} ({om[r]}), tol {tol[r]}")
        near[r] = True
        stats["ids_differ"] += 1

    gn = np.asarray(gpu["n_accepted"], np.int64)
    own = accept_from(gi, drafts, R, T)
    assert np.array_equal(gn, own), f"n_accepted {gn} != prefix from GPU ids {own}"
    on = np.asarray(orc["n_accepted"], np.int64)
    for i in range(R):
        if gn[i] != on[i]:
            first = i * T + min(gn[i], on[i])
            assert near[first], f"request {i}: n_accepted {gn[i]} vs {on[i]} without a near tie"
            stats["accept_divergence"] += 1
    return stats

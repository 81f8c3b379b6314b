"""CPU oracle of verification through a draft-vocabulary head: a head whose
rows are a subset of the vocabulary, with a row -> token id map.

TEST INFRASTRUCTURE ONLY: imported by the test suite and the benchmark's
CPU-baseline leg, never by the GPU library or its binding.

The draft vocabulary is from "HyperQwen: 1,000 tok/s on a Single RTX 3090
Through Aggressive Recurrent-State Speculation", Technical Insight (the
speculation configuration cuts the drafter's vocabulary to the 8192 tokens
actually observed, out of about 152k) and the HyperQwen README, "Roadmap"
(a 40k-token draft vocabulary).  The pages do not say how a row subset is
addressed; the reading used here: the head holds the rows of the subset in
increasing token order, vocab_ids[row] is the token id of each row
(strictly increasing, non-negative), the greedy argmax is taken over the
head's rows with the lowest row winning ties (the lowest token id, since
the map increases), the reported id is vocab_ids[argmax row], and drafted
token ids are compared with those reported ids.  Logits are indexed by row.
Every number comes from the pinned verify oracle (oracle.py / oracle.c); this
module only applies the map.
"""
from __future__ import annotations

import numpy as np

from . import oracle


def count_bad_map(vocab_ids) -> int:
    """Positions where the map is not strictly increasing and non-negative."""
    m = np.asarray(vocab_ids, np.int64)
    if m.size == 0:
        return 0
    return int(m[0] < 0) + int(np.sum(m[1:] <= m[:-1]))


def verify_mapped(hidden_bits, packed, scales_bits, vocab_ids, draft_ids, R: int, T: int, V: int,
                  H: int, want_logits: bool = False, n_threads: int = 0) -> dict:
    """Verify step through a row-subset head.  Returns the verify oracle's
    dict with argmax_ids replaced by token ids (argmax_rows keeps the head
    rows) and n_accepted counted against the token ids."""
    vmap = np.ascontiguousarray(vocab_ids, np.int32)
    if vmap.shape != (V,):
        raise ValueError("vocab_ids must hold one id per head row")
    if count_bad_map(vmap):
        raise ValueError("vocab_ids must be strictly increasing and non-negative")
    o = oracle.verify(hidden_bits, packed, scales_bits, np.zeros((R, max(T - 1, 0)), np.int32),
                      R, T, V, H, want_logits=want_logits, n_threads=n_threads)
    rows = o["argmax_ids"]
    ids = vmap[rows].astype(np.int32)
    out = dict(o)
    out["argmax_rows"] = rows
    out["argmax_ids"] = ids
    out["n_accepted"] = oracle.accept(ids, draft_ids, R, T)
    return out

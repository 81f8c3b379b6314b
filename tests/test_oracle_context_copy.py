"""Pins of the context-copy drafter oracle (oracle/context_copy.py): hand
cases written out from the definition, brute force over every end position
and length on small random inputs, and the invariants of a proposal."""
import numpy as np

from oracle import context_copy as cc


def test_hand_cases():
    #          0  1  2  3  4  5  6  7  8  9 10 11
    prompt = [5, 6, 7, 8, 9, 5, 6, 7, 1, 2, 3, 4]
    # key ends with 5 6 7: matches end at e=3 (5 6 7 | 8) and e=8 (5 6 7 | 1);
    # both of length 3 (the 4th key token 0 matches neither) -> the latest, e=8
    r = cc.propose(prompt, [0, 5, 6, 7], n_min=1, n_out=8)
    assert (r["match_end"], r["match_len"], r["count"]) == (8, 3, 4)
    assert r["tokens"].tolist() == [1, 2, 3, 4]
    # key 9 5 6 7: only e=8 matches all four (prompt[4..7] = 9 5 6 7)
    r = cc.propose(prompt, [9, 5, 6, 7], n_min=1, n_out=2)
    assert (r["match_end"], r["match_len"], r["tokens"].tolist()) == (8, 4, [1, 2])
    # key ... 8: the longest match is one token, at e=4 (prompt[3] = 8)
    r = cc.propose(prompt, [1, 1, 8], n_min=1, n_out=8)
    assert (r["match_end"], r["match_len"], r["tokens"].tolist()) == (4, 1, [9, 5, 6, 7, 1, 2, 3, 4])
    # n_min filters it out
    r = cc.propose(prompt, [1, 1, 8], n_min=2, n_out=8)
    assert (r["match_end"], r["count"], r["match_len"]) == (-1, 0, 0)
    # a match ending at the last prompt token proposes nothing there: key ...3 4
    # matches only at e=12 (no following token), so no proposal
    r = cc.propose(prompt, [3, 4], n_min=1, n_out=8)
    assert r["count"] == 0
    # no match at all
    assert cc.propose(prompt, [99, 98], n_min=1, n_out=8)["count"] == 0


def brute(prompt, key, n_min, n_out):
    L, n = len(prompt), len(key)
    best_len, best_e = 0, -1
    for e in range(1, L):                 # at least one token follows
        ell = 0
        while ell < n and ell < e and prompt[e - 1 - ell] == key[n - 1 - ell]:
            ell += 1
        if ell >= n_min and (ell > best_len or (ell == best_len and e > best_e)):
            best_len, best_e = ell, e
    if best_e < 0:
        return [], -1, 0
    return list(prompt[best_e:best_e + min(n_out, L - best_e)]), best_e, best_len


def test_brute_force_small_vocab():
    rng = np.random.default_rng(0)
    for trial in range(400):
        L = int(rng.integers(1, 60))
        vocab = int(rng.integers(2, 6))       # small vocabulary: many partial matches
        prompt = rng.integers(0, vocab, size=L).tolist()
        n_max = int(rng.integers(1, 9))
        key = rng.integers(0, vocab, size=n_max).tolist()
        n_min = int(rng.integers(1, n_max + 1))
        n_out = int(rng.integers(1, 10))
        r = cc.propose(prompt, key, n_min, n_out)
        toks, e, ell = brute(prompt, key, n_min, n_out)
        assert (r["tokens"].tolist(), r["match_end"], r["match_len"]) == (toks, e, ell), (prompt, key)


def test_proposal_invariants():
    rng = np.random.default_rng(1)
    prompt = rng.integers(0, 151936, size=25000)
    start = 12345
    key = prompt[start - 16:start].copy()         # the answer is quoting the prompt
    r = cc.propose(prompt, key, n_min=2, n_out=8)
    assert r["match_end"] == start and r["match_len"] == 16
    assert np.array_equal(r["tokens"], prompt[start:start + 8])
    # the matched span really is the key's suffix
    e, ell = r["match_end"], r["match_len"]
    assert np.array_equal(prompt[e - ell:e], key[16 - ell:])
    key2 = key.copy()
    key2[10] = -1                                  # a drafted token that breaks the quote
    r2 = cc.propose(prompt, key2, n_min=2, n_out=8)
    assert r2["match_end"] == start and r2["match_len"] == 5

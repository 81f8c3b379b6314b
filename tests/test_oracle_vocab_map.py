"""Pins of the draft-vocabulary oracle (oracle/vocab_map.py): against the
full-vocabulary oracle restricted to the subset with numpy's argmax, the
identity map, the map checks and acceptance in token space."""
import numpy as np
import pytest

from int4_output_head_amd import synth
from oracle import vocab_map as vm


def test_identity_map_is_plain_verify(oracle_mod):
    V, H, T = 300, 64, 4
    inp = synth.uniform_inputs(T, V, H, seed=1)
    plain = oracle_mod.verify(inp["hidden"], inp["packed"], inp["scales"], np.zeros(T - 1, np.int32),
                              1, T, V, H)
    d = np.asarray(plain["argmax_ids"][: T - 1], np.int32)
    o = vm.verify_mapped(inp["hidden"], inp["packed"], inp["scales"], np.arange(V), d, 1, T, V, H)
    assert np.array_equal(o["argmax_ids"], plain["argmax_ids"])
    assert np.array_equal(o["logits_max"], plain["logits_max"])
    assert int(o["n_accepted"][0]) == T - 1


def test_subset_head_equals_full_head_restricted(oracle_mod):
    """The sub-head's mapped argmax is the full head's argmax over the subset
    (numpy argmax of the full logits restricted to the subset, first
    occurrence on ties)."""
    Vf, H, T = 1000, 96, 3
    inp = synth.int_exact_inputs(T, Vf, H, seed=7)          # many exact ties
    full = oracle_mod.logits(inp["hidden"], inp["packed"], inp["scales"], T, Vf, H)
    rng = np.random.default_rng(3)
    S = np.sort(rng.choice(Vf, 137, replace=False)).astype(np.int32)
    o = vm.verify_mapped(inp["hidden"], inp["packed"][S], inp["scales"], S,
                         np.zeros(T - 1, np.int32), 1, T, len(S), H, want_logits=True)
    want = S[np.argmax(full[:, S], axis=1)]
    assert np.array_equal(o["argmax_ids"], want)
    assert np.array_equal(o["logits"], full[:, S])
    assert np.array_equal(o["logits_max"], full[np.arange(T), want])


def test_acceptance_uses_token_ids(oracle_mod):
    V, H, T = 50, 32, 5
    inp = synth.uniform_inputs(T, V, H, seed=2)
    vmap = (np.arange(V) * 3 + 11).astype(np.int32)
    o = vm.verify_mapped(inp["hidden"], inp["packed"], inp["scales"], vmap, np.zeros(T - 1, np.int32),
                         1, T, V, H)
    ids, rows = o["argmax_ids"], o["argmax_rows"]
    assert np.array_equal(ids, vmap[rows])
    good = np.asarray(ids[: T - 1], np.int32)
    assert int(vm.verify_mapped(inp["hidden"], inp["packed"], inp["scales"], vmap, good, 1, T, V,
                                H)["n_accepted"][0]) == T - 1
    # the head rows themselves are not token ids: drafting rows is rejected at once
    as_rows = np.asarray(rows[: T - 1], np.int32)
    assert int(vm.verify_mapped(inp["hidden"], inp["packed"], inp["scales"], vmap, as_rows, 1, T, V,
                                H)["n_accepted"][0]) == 0
    bad2 = good.copy()
    bad2[2] = (bad2[2] + 1)
    assert int(vm.verify_mapped(inp["hidden"], inp["packed"], inp["scales"], vmap, bad2, 1, T, V,
                                H)["n_accepted"][0]) == 2


def test_map_checks():
    assert vm.count_bad_map([0, 1, 5, 9]) == 0
    assert vm.count_bad_map([-1, 1, 5, 9]) == 1
    assert vm.count_bad_map([0, 1, 1, 9]) == 1
    assert vm.count_bad_map([3, 2, 1, 0]) == 3
    with pytest.raises(ValueError):
        vm.verify_mapped(np.zeros((1, 32), np.uint16), np.zeros((2, 16), np.uint8),
                         np.zeros(32, np.uint16), [1, 1], None, 1, 1, 2, 32)

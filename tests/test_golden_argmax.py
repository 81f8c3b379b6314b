"""The stored oracle argmax files (written by tests/golden/make_argmax.py,
which calls only the oracle) agree with fresh oracle runs."""
import json
import os

import numpy as np
import pytest

from int4_output_head_amd import synth

HERE = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(HERE, f"argmax_{name}.json")) as f:
        return json.load(f)


@pytest.mark.parametrize("name,trials", [("tiny", [0]), ("draft_vocab", [0, 1, 999]),
                                         ("full_t16", [0]), ("shard_t16", [0, 19]),
                                         ("two_blocks_t16", [9])])
def test_stored_argmax_matches_oracle(oracle_mod, name, trials):
    cfg = synth.CONFIGS[name]
    data = _load(name)
    assert (data["V"], data["H"], data["R"], data["T"]) == (cfg.V, cfg.H, cfg.R, cfg.T)
    head = synth.make_head(cfg)
    for t in trials:
        x = synth.make_hidden(cfg, t)
        lg = oracle_mod.logits(x, head["packed"], head["scales"], cfg.M, cfg.V, cfg.H)
        idx, _, gap, amax = oracle_mod.argmax_rows(lg)
        rec = data["trials"][str(t)]
        assert idx.tolist() == rec["argmax"]
        assert np.allclose(gap, rec["gap"]) and np.allclose(amax, rec["amax"])


def test_stored_batch_argmax_rows_match_oracle(oracle_mod):
    """The 64 x 4 batch file, checked on a few rows of two trials (the whole
    file takes the oracle minutes)."""
    cfg = synth.CONFIGS["batch"]
    data = _load("batch")
    assert (data["V"], data["H"], data["R"], data["T"]) == (cfg.V, cfg.H, cfg.R, cfg.T)
    head = synth.make_head(cfg)
    rows = [0, 101, 255]
    for t in (0, 4):
        x = synth.make_hidden(cfg, t).reshape(cfg.M, cfg.H)
        lg = oracle_mod.logits(np.ascontiguousarray(x[rows]), head["packed"], head["scales"],
                               len(rows), cfg.V, cfg.H)
        idx, _, gap, amax = oracle_mod.argmax_rows(lg)
        rec = data["trials"][str(t)]
        assert idx.tolist() == [rec["argmax"][r] for r in rows]
        assert np.allclose(gap, [rec["gap"][r] for r in rows])
        assert np.allclose(amax, [rec["amax"][r] for r in rows])

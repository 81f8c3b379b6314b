"""GPU parity on every seeded trial of the multi-trial workloads: the 1000
repeats of the draft-vocabulary decode (V=8192, H=5120, T=1), the 20 trials
of the full-vocabulary T=8 and T=16 verify blocks, the 5 trials of the
64 x 4 batch, the 20 trials of one GPU's vocabulary shard (V=18992, T=16),
and the 10 trials of two wide verify blocks at once (2 x T=16 = 32 rows).  Each GPU argmax is compared with the oracle's stored argmax
(tests/golden/argmax_*.json, written by a script that calls only the
oracle) under the near-tie rule: where the ids differ, the oracle logit at
the GPU's id, recomputed for that one entry, must lie within
2e-3 * max_v |oracle logit| (stored) of the oracle's maximum.  n_accepted
must equal the prefix recomputed from the GPU's own ids exactly, and the
oracle's (from the stored argmax and the same drafts) unless the first
difference is a near-tie row.  Needs an MI355X and the built library.
"""
import json
import os
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from int4_output_head_amd import synth  # noqa: E402

from . import parity  # noqa: E402

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def say(msg):
    print(f"[gpu-trials] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def vh():
    from int4_output_head_amd import binding
    binding.load_library()
    assert torch.cuda.is_available(), "no GPU visible"
    return binding


@pytest.mark.parametrize("name", ["draft_vocab", "full_t8", "full_t16", "batch", "shard_t16", "two_blocks_t16"])
def test_every_stored_trial(vh, oracle_mod, name):
    cfg = synth.CONFIGS[name]
    with open(os.path.join(GOLDEN, f"argmax_{name}.json")) as f:
        stored = json.load(f)
    assert (stored["V"], stored["H"], stored["R"], stored["T"]) == (cfg.V, cfg.H, cfg.R, cfg.T)
    assert len(stored["trials"]) == cfg.trials
    say(f"{name}: {cfg.trials} trials, M={cfg.M} V={cfg.V} H={cfg.H}")
    head = synth.make_head(cfg)
    w = torch.from_numpy(head["packed"]).cuda()
    s = torch.from_numpy(head["scales"]).view(torch.float16).cuda()
    ws = vh.Workspace(vh.workspace_bytes(cfg.R, cfg.T, cfg.V, cfg.H), w.device)
    totals = dict(rows=0, near_tie_rows=0, ids_differ=0, accept_divergence=0)
    for trial in range(cfg.trials):
        rec = stored["trials"][str(trial)]
        ids = np.array(rec["argmax"], np.int32)
        x = synth.make_hidden(cfg, trial)
        drafts = (synth.finalize_drafts(cfg, synth.draft_plan(cfg, trial), ids) if cfg.T > 1 else None)
        xt = torch.from_numpy(x).view(torch.float16).cuda().reshape(cfg.R, cfg.T, cfg.H)
        dt = torch.from_numpy(drafts).cuda() if drafts is not None else None
        lmax, amax_ids, nacc = vh.verify_batch(xt, w, s, dt, workspace=ws)
        torch.cuda.synchronize()
        gi = amax_ids.cpu().numpy()

        def orc_logit(r, v):
            return float(oracle_mod.logit_one(x[r], head["packed"][v], head["scales"], cfg.H))
        # the oracle's maximum per row: its logit at its own argmax (one dot each)
        om = np.array([orc_logit(r, int(ids[r])) for r in range(cfg.M)], np.float32)
        orc = dict(logits_max=om, argmax_ids=ids, gap=np.array(rec["gap"], np.float32),
                   amax=np.array(rec["amax"], np.float32),
                   n_accepted=parity.accept_from(ids, drafts, cfg.R, cfg.T))
        g = dict(logits_max=lmax.cpu().numpy(), argmax_ids=gi, n_accepted=nacc.cpu().numpy())
        st = parity.check(g, orc, cfg.R, cfg.T, drafts, orc_logit_at=orc_logit)
        for k in totals:
            totals[k] += st[k]
    say(f"{name}: {totals}")
    assert totals["rows"] == cfg.M * cfg.trials

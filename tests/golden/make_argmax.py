"""Writes the oracle's greedy argmax ids of every seeded trial of the named
workloads to tests/golden/argmax_<name>.json.  It calls only the oracle and
the seeded input generator; the benchmark reads these files to build draft
ids that agree with the target's argmax, and the tests check the files
against fresh oracle runs.

    python tests/golden/make_argmax.py full_t16 full_t8 tiny draft_vocab batch shard_t16 two_blocks_t16
"""
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

from int4_output_head_amd import synth  # noqa: E402
from oracle import oracle  # noqa: E402


def main(names):
    for name in names:
        cfg = synth.CONFIGS[name]
        t0 = time.time()
        head = synth.make_head(cfg)
        out = dict(config=name, V=cfg.V, H=cfg.H, R=cfg.R, T=cfg.T, head_seed=0, trials={})
        for trial in range(cfg.trials):
            x = synth.make_hidden(cfg, trial)
            lg = oracle.logits(x, head["packed"], head["scales"], cfg.M, cfg.V, cfg.H)
            idx, mx, gap, amax = oracle.argmax_rows(lg)
            out["trials"][str(trial)] = dict(argmax=idx.tolist(), gap=[float(g) for g in gap],
                                             amax=[float(a) for a in amax])
            print(f"{name} trial {trial} done {time.time() - t0:.1f}s", flush=True)
        with open(os.path.join(HERE, f"argmax_{name}.json"), "w") as f:
            json.dump(out, f)


if __name__ == "__main__":
    main(sys.argv[1:] or ["tiny", "draft_vocab", "full_t8", "full_t16", "batch", "shard_t16", "two_blocks_t16"])

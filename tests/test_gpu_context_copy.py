"""GPU parity of the context-copy drafter (context_copy_propose) against the
oracle (oracle/context_copy.py): integer work, bit-exact.  Needs an MI355X
and the built library."""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from int4_output_head_amd import synth  # noqa: E402
from oracle import context_copy as cc  # noqa: E402

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu-context-copy] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def vh():
    from int4_output_head_amd import binding
    binding.load_library()
    assert torch.cuda.is_available(), "no GPU visible"
    return binding


def run(vh, prompts, keys, n_min, n_out):
    flat = np.concatenate([np.asarray(p, np.int32) for p in prompts]) if prompts else np.zeros(0, np.int32)
    offs = np.zeros(len(prompts) + 1, np.int64)
    offs[1:] = np.cumsum([len(p) for p in prompts])
    if flat.size == 0:
        flat = np.zeros(1, np.int32)
    out = vh.context_copy(torch.from_numpy(flat).cuda(), torch.from_numpy(offs).cuda(),
                          torch.from_numpy(np.asarray(keys, np.int32)).cuda(), n_min=n_min, n_out=n_out)
    torch.cuda.synchronize()
    tok, cnt, end, ln = (t.cpu().numpy() for t in out)
    for r, (p, k) in enumerate(zip(prompts, keys)):
        o = cc.propose(p, k, n_min, n_out)
        assert (int(cnt[r]), int(end[r]), int(ln[r])) == (o["count"], o["match_end"], o["match_len"]), r
        assert tok[r, : o["count"]].tolist() == o["tokens"].tolist(), r
        assert np.all(tok[r, o["count"]:] == -1)
    return cnt, end, ln


def test_small_vocab_random(vh):
    """Many partial matches and ties (small vocabulary), ragged lengths,
    empty and one-token prompts."""
    rng = np.random.default_rng(0)
    prompts, keys = [], []
    for r in range(300):
        L = int(rng.choice([0, 1, 2, 3, 17, 100, 1023, 1024, 1025, 5000]))
        prompts.append(rng.integers(0, 4, size=L).tolist())
        keys.append(rng.integers(0, 4, size=12).tolist())
    for n_min, n_out in ((1, 8), (3, 8), (12, 5), (2, 64)):
        say(f"small vocab n_min={n_min} n_out={n_out}")
        run(vh, prompts, keys, n_min, n_out)


def test_quoting_workload(vh):
    """The context-copy workload: 25,000-token prompts; the key ends with a
    passage of the prompt (quoting, as in document reproduction), with the
    drafted tail broken in some requests and no quote at all in others."""
    rng = np.random.default_rng(1)
    R, L, n_max = 64, 25000, 16
    prompts, keys, want_end = [], [], []
    for r in range(R):
        p = rng.integers(0, 151936, size=L)
        s = int(rng.integers(n_max, L - 1))
        k = p[s - n_max:s].copy()
        c = rng.random()
        if c < 0.2:
            k[int(rng.integers(0, n_max))] = 151936 + r      # a draft that leaves the quote
        elif c < 0.3:
            k[-1] = 151936 + r                                # no match of the last token
        prompts.append(p)
        keys.append(k)
    cnt, end, ln = run(vh, prompts, keys, 2, 8)
    say(f"quoting: matches {int((cnt > 0).sum())} of {R}, full-length {int((ln == n_max).sum())}")


def test_repeated_passages_pick_latest(vh):
    """A passage that occurs several times: the latest occurrence wins."""
    rng = np.random.default_rng(2)
    p = rng.integers(0, 1000, size=20000)
    passage = rng.integers(0, 1000, size=20)
    for at in (100, 7000, 15000):
        p[at:at + 20] = passage
    key = passage[-16:]
    cnt, end, ln = run(vh, [p.tolist()], [key.tolist()], 1, 8)
    assert int(end[0]) == 15020 and int(ln[0]) == 16

"""GPU parity of verification through a draft-vocabulary head
(verify_lm_head_int4_mapped) against the oracle (oracle/vocab_map.py), on
both kernel paths.  Needs an MI355X and the built library."""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from int4_output_head_amd import synth  # noqa: E402
from oracle import vocab_map as vm  # noqa: E402

from . import parity  # noqa: E402

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu-vocab-map] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def vh():
    from int4_output_head_amd import binding
    binding.load_library()
    assert torch.cuda.is_available(), "no GPU visible"
    return binding


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.cuda()


def vocab_subset(V, V_full, seed):
    rng = np.random.default_rng(seed)
    return np.sort(rng.choice(V_full, V, replace=False)).astype(np.int32)


def run_case(vh, oracle_mod, inp, vmap, R, T, V, H, logits=True):
    o0 = vm.verify_mapped(inp["hidden"], inp["packed"], inp["scales"], vmap,
                          np.zeros((R, max(T - 1, 0)), np.int32), R, T, V, H)
    drafts = np.asarray(o0["argmax_ids"], np.int32).reshape(R, T)[:, : T - 1].copy()
    if T > 2:
        drafts[:, T // 2] = drafts[:, T // 2] + 1              # a token id that is not the argmax
    o = vm.verify_mapped(inp["hidden"], inp["packed"], inp["scales"], vmap, drafts, R, T, V, H,
                         want_logits=True)
    out = vh.verify_mapped(dev(inp["hidden"], torch.float16).reshape(R, T, H), dev(inp["packed"]),
                           dev(inp["scales"], torch.float16), dev(vmap),
                           None if T == 1 else dev(drafts), logits=logits)
    torch.cuda.synchronize()
    ids = out[1].cpu().numpy()
    # token ids back to head rows (the map is strictly increasing) for the
    # row-indexed parity rule; every returned id must be a mapped token
    rows = np.searchsorted(vmap, ids)
    assert np.all(rows < V) and np.array_equal(vmap[rows], ids)
    g = dict(logits_max=out[0].cpu().numpy(), argmax_ids=rows, n_accepted=out[2].cpu().numpy())
    if logits:
        g["logits"] = out[3].cpu().numpy()
    orow = dict(o)
    orow["argmax_ids"] = o["argmax_rows"]
    # drafts in row space (-1 for a token outside the head: never matches),
    # an exact image of the token-space comparison since the map is injective
    drows = None
    if T > 1:
        pos = np.minimum(np.searchsorted(vmap, drafts), V - 1)
        drows = np.where(vmap[pos] == drafts, pos, -1).astype(np.int32)
    st = parity.check(g, orow, R, T, drows)
    # acceptance in token space, from the GPU's own ids and against the oracle
    assert np.array_equal(out[2].cpu().numpy(), parity.accept_from(ids, drafts, R, T))
    if st["ids_differ"] == 0:
        assert np.array_equal(out[2].cpu().numpy(), o["n_accepted"])
        assert np.array_equal(ids, o["argmax_ids"])
    return st


@pytest.mark.parametrize("R,T,V,H", [(1, 1, 8192, 5120), (1, 8, 3001, 1024), (1, 16, 40000, 256),
                                     (4, 4, 517, 96), (64, 4, 2048, 512), (3, 9, 1000, 160)])
def test_mapped_parity(vh, oracle_mod, R, T, V, H):
    say(f"mapped R={R} T={T} V={V} H={H}")
    inp = synth.uniform_inputs(R * T, V, H, seed=R + T + V + H)
    vmap = vocab_subset(V, 151936, seed=V)
    st = run_case(vh, oracle_mod, inp, vmap, R, T, V, H)
    say(f"stats {st}")


def test_mapped_int_exact_ties(vh, oracle_mod):
    """Exact ties: the lowest row (= lowest token id) wins on both paths."""
    for R, T in ((1, 8), (8, 4)):
        V, H = 2000, 512
        inp = synth.int_exact_inputs(R * T, V, H, seed=5)
        vmap = vocab_subset(V, 151936, seed=1)
        run_case(vh, oracle_mod, inp, vmap, R, T, V, H)


def test_identity_map_equals_unmapped(vh):
    R, T, V, H = 2, 8, 5000, 640
    inp = synth.uniform_inputs(R * T, V, H, seed=9)
    x = dev(inp["hidden"], torch.float16).reshape(R, T, H)
    w = dev(inp["packed"])
    s = dev(inp["scales"], torch.float16)
    d = dev(np.random.default_rng(0).integers(0, V, size=(R, T - 1)).astype(np.int32))
    a = vh.verify_batch(x, w, s, d, logits=True)
    b = vh.verify_mapped(x, w, s, dev(np.arange(V, dtype=np.int32)), d, logits=True)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u, v)


def test_check_vocab_map(vh):
    good = np.arange(0, 3 * 70000, 3, dtype=np.int32)
    assert int(vh.check_vocab_map(dev(good)).item()) == 0
    bad = good.copy()
    bad[0] = -5
    bad[100] = bad[99]
    bad[5000] = bad[4998]
    # map[0] < 0; map[100] == map[99]; map[5000] < map[4999]
    assert int(vh.check_vocab_map(dev(bad)).item()) == vm.count_bad_map(bad) == 3

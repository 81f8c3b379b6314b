"""GPU parity of the offline requantisation (include/int4vh_requant.h) against
the requantisation oracle (oracle/requant.py): scales, codes and packed bytes
are integers or bit patterns, so the bar is bit-exact.  Needs an MI355X and
the built library."""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from int4_output_head_amd import synth  # noqa: E402
from oracle import requant as rq  # noqa: E402

pytestmark = pytest.mark.gpu

TDT = {"f16": torch.float16, "bf16": torch.bfloat16}
ODT = {"f16": rq.F16, "bf16": rq.BF16}


def say(msg):
    print(f"[gpu-requant] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def vh():
    from int4_output_head_amd import binding
    binding.load_library()
    assert torch.cuda.is_available(), "no GPU visible"
    return binding


def dev_bits(bits, dtype):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(dtype).cuda()


def host_bits(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("N,H,dt", [(1, 32, "f16"), (7, 96, "bf16"), (129, 544, "f16"),
                                    (300, 5120, "bf16"), (4096, 5120, "f16"), (513, 8192, "f16")])
def test_amax_matches_oracle(vh, N, H, dt):
    say(f"amax N={N} H={H} {dt}")
    inp = synth.requant_inputs(1, H, N, seed=N + H, w_dtype=dt, a_dtype=dt)
    a = dev_bits(inp["acts"], TDT[dt])
    got = vh.requant_amax(a)
    torch.cuda.synchronize()
    want = rq.calib_amax(inp["acts"], ODT[dt])
    assert np.array_equal(got.cpu().numpy().view(np.uint32), want.view(np.uint32))


def test_amax_accumulates_over_batches(vh):
    H = 640
    inp = synth.requant_inputs(1, H, 700, seed=11)
    a = dev_bits(inp["acts"], torch.float16)
    amax = vh.requant_amax(a[:300])
    vh.requant_amax(a[300:301], amax, accumulate=True)
    vh.requant_amax(a[301:], amax, accumulate=True)
    torch.cuda.synchronize()
    want = rq.calib_amax(inp["acts"], rq.F16)
    assert np.array_equal(amax.cpu().numpy().view(np.uint32), want.view(np.uint32))
    # a fresh (non-accumulating) call forgets the earlier batches
    vh.requant_amax(a[:5], amax)
    torch.cuda.synchronize()
    want5 = rq.calib_amax(inp["acts"][:5], rq.F16)
    assert np.array_equal(amax.cpu().numpy().view(np.uint32), want5.view(np.uint32))


def test_scales_match_oracle(vh):
    rng = np.random.default_rng(7)
    H = 4096
    amax = np.concatenate([
        np.zeros(32), rng.uniform(0, 1e-7, 256), rng.lognormal(0, 3, 3000),
        np.array([65504 * 7.0, 65519.9 * 7, 65520 * 7.0, 1e30, 3.4e38]),
        rng.uniform(1, 100, H - 3293)]).astype(np.float32)
    assert amax.size == H
    got = vh.requant_scales(torch.from_numpy(amax).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(got), rq.scales_from_amax(amax))


def _pack_case(vh, W_bits, s_bits, dt):
    W = dev_bits(W_bits, TDT[dt])
    s = dev_bits(s_bits, torch.float16)
    got = vh.requant_pack(W, s)
    torch.cuda.synchronize()
    want = rq.pack(rq.quantize(W_bits, ODT[dt], s_bits))
    g = got.cpu().numpy()
    bad = np.argwhere(g != want)
    assert bad.size == 0, f"{len(bad)} bytes differ, first at {bad[:3].tolist()}"
    return g


@pytest.mark.parametrize("V,H,dt", [(1, 32, "f16"), (3, 64, "bf16"), (17, 96, "f16"),
                                    (1000, 5120, "f16"), (333, 8192, "bf16"), (257, 160, "f16"),
                                    (4099, 1024, "bf16")])
def test_pack_matches_oracle(vh, V, H, dt):
    say(f"pack V={V} H={H} {dt}")
    inp = synth.requant_inputs(V, H, 64, seed=V * 7 + H, w_dtype=dt, a_dtype="f16")
    s = rq.scales_from_amax(rq.calib_amax(inp["acts"], rq.F16))
    _pack_case(vh, inp["W"], s, dt)


def test_pack_exact_ties_and_special_scales(vh):
    """Weights exactly on a rounding boundary (k + 1/2) * s go to the even
    code; scales of 0, subnormal and infinity; weights far beyond the range;
    weights one binary16 step either side of a boundary."""
    rng = np.random.default_rng(3)
    V, H = 64, 512
    m = rng.integers(1, 64, size=H)
    s = (m * 2.0 ** -12)                                     # few significant bits
    s[:8] = 0.0
    s[8:16] = np.inf
    s[16:24] = 2.0 ** -24 * rng.integers(1, 8, size=8)       # binary16 subnormals
    k = rng.integers(-9, 9, size=(V, H))
    W = (k + 0.5) * np.where(np.isfinite(s), s, 1.0)         # exact in binary16
    Wb = synth.f16_bits(W)
    assert np.array_equal(Wb.view(np.float16).astype(np.float64)[:, 24:], W[:, 24:])
    # rows 32..47: one binary16 step above, rows 48..63: one step below
    Wb[32:48] = np.where(Wb[32:48] & 0x7FFF, Wb[32:48] + 1, Wb[32:48])
    Wb[48:56] = np.where(Wb[48:56] & 0x7FFF, Wb[48:56] - 1, Wb[48:56])
    Wb[56, :] = synth.f16_bits(np.full(H, 65504.0))
    Wb[57, :] = synth.f16_bits(np.full(H, -65504.0))
    Wb[58, :] = synth.f16_bits(np.zeros(H)) | 0x8000          # -0.0
    sb = synth.f16_bits(s)
    got = _pack_case(vh, Wb, sb, "f16")
    q = rq.quantize(Wb, rq.F16, sb)
    assert np.all(q[:, :8] == 0) and np.all(q[:, 8:16] == 0)
    # on the exact boundaries the codes are even (or clamped)
    tie_rows = q[:32, 24:]
    assert np.all((tie_rows % 2 == 0) | (np.abs(tie_rows) == 7))
    assert got.shape == (V, H // 2)


def test_pack_bf16_extremes(vh):
    rng = np.random.default_rng(5)
    V, H = 40, 256
    W = rng.standard_normal((V, H)) * np.exp(rng.uniform(-60, 60, size=(V, H)))
    s = synth.f16_bits(rng.lognormal(-4, 2, size=H))
    _pack_case(vh, synth.bf16_bits(W), s, "bf16")


def test_requantize_one_call_equals_steps(vh):
    V, H, N = 999, 1536, 333
    inp = synth.requant_inputs(V, H, N, seed=21, w_dtype="bf16", a_dtype="bf16")
    W = dev_bits(inp["W"], torch.bfloat16)
    a = dev_bits(inp["acts"], torch.bfloat16)
    packed, scales, amax = vh.requantize(W, a)
    torch.cuda.synchronize()
    want_packed, want_s = rq.requantize(inp["W"], rq.BF16, inp["acts"], rq.BF16)
    assert np.array_equal(host_bits(scales), want_s)
    assert np.array_equal(packed.cpu().numpy(), want_packed)
    assert np.array_equal(amax.cpu().numpy(), rq.calib_amax(inp["acts"], rq.BF16))


def test_full_size_head_sampled_rows(vh):
    """The full-vocabulary head (V=151936, H=5120, binary16), packed in the
    launch configuration the benchmark times; 3000 sampled rows against the
    oracle, and no illegal nibble anywhere."""
    V, H, N = 151936, 5120, 4096
    say("full-size requantisation: generating inputs")
    inp = synth.requant_inputs(V, H, N, seed=0)
    W = dev_bits(inp["W"], torch.float16)
    a = dev_bits(inp["acts"], torch.float16)
    say("full-size requantisation: GPU")
    packed, scales, _ = vh.requantize(W, a)
    nbad = vh.check_weights(packed)
    torch.cuda.synchronize()
    assert int(nbad.item()) == 0
    s_want = rq.scales_from_amax(rq.calib_amax(inp["acts"], rq.F16))
    assert np.array_equal(host_bits(scales), s_want)
    rows = np.sort(np.random.default_rng(1).choice(V, 3000, replace=False))
    rows = np.concatenate([[0, 1, V - 2, V - 1], rows])
    want = rq.pack(rq.quantize(inp["W"][rows], rq.F16, s_want))
    got = packed[torch.from_numpy(rows).cuda()].cpu().numpy()
    assert np.array_equal(got, want)


def test_requantized_head_verifies_like_oracle(vh, oracle_mod):
    """Closure: a head requantised on the GPU, verified on the GPU, against
    the oracle's requantisation verified by the oracle."""
    V, H, N, T = 3000, 1024, 256, 8
    inp = synth.requant_inputs(V, H, N, seed=4)
    packed_o, s_o = rq.requantize(inp["W"], rq.F16, inp["acts"], rq.F16)
    W = dev_bits(inp["W"], torch.float16)
    a = dev_bits(inp["acts"], torch.float16)
    packed, scales, _ = vh.requantize(W, a)
    x = synth.f16_bits(np.random.default_rng(9).standard_normal((T, H)))
    o = oracle_mod.verify(x, packed_o, s_o, np.zeros((1, T - 1), np.int32), 1, T, V, H)
    drafts = np.asarray(o["argmax_ids"][: T - 1], np.int32)
    drafts[5] = (drafts[5] + 1) % V
    o = oracle_mod.verify(x, packed_o, s_o, drafts[None, :], 1, T, V, H, want_logits=True)
    lmax, ids, nacc, lg = vh.verify(dev_bits(x, torch.float16), packed, scales,
                                    torch.from_numpy(drafts).cuda(), logits=True)
    torch.cuda.synchronize()
    assert np.array_equal(packed.cpu().numpy(), packed_o)
    from . import parity
    g = dict(logits_max=lmax.cpu().numpy(), argmax_ids=ids.cpu().numpy(),
             n_accepted=nacc.cpu().numpy(), logits=lg.cpu().numpy())
    parity.check(g, o, 1, T, drafts[None, :])
    assert int(nacc.item()) == int(o["n_accepted"][0]) == 5

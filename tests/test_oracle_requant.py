"""Pins of the requantisation oracle (oracle/requant.py) against what the
definition and the mathematics fix: hand-derived roundings, exact rational
arithmetic, the dequantisation error bound, round trips, and the verify
oracle's own (pinned) unpacking of the packed head."""
from fractions import Fraction

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import requant as rq  # noqa: E402


def f16(vals):
    return np.asarray(vals, np.float64).astype(np.float16).view(np.uint16)


def test_round_half_even_and_clamp_hand_cases():
    # s = 1 exactly, so W / s = W with no division rounding; expected values
    # written out from the definition: round half to even, then clamp to +-7
    w = [0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 6.5, 7.5, -7.5, 8.0, -100.0, 3.49, 3.51, 0.0, -0.25]
    want = [0, 2, 2, 0, -2, -2, 6, 7, -7, 7, -7, 3, 4, 0, 0]
    q = rq.quantize(f16(w)[None, :], rq.F16, f16([1.0] * len(w)))
    assert q[0].tolist() == want


def test_exact_rational_rounding():
    """On random weights and scales the binary32 quotient decides the same
    integer as the exact rational quotient, except within a hair of a tie."""
    rng = np.random.default_rng(1)
    w = f16(rng.normal(0, 0.05, size=(64, 64)))
    s = f16(rng.lognormal(-5, 0.5, size=64))
    q = rq.quantize(w, rq.F16, s)
    wv = w.view(np.float16).astype(np.float64)
    sv = s.view(np.float16).astype(np.float64)
    near_tie = 0
    for v in range(64):
        for h in range(64):
            exact = Fraction(float(wv[v, h])) / Fraction(float(sv[h]))
            fl = exact.numerator // exact.denominator
            frac = exact - fl
            if abs(frac - Fraction(1, 2)) < Fraction(1, 1 << 20) * (abs(exact) + 1):
                near_tie += 1
                continue
            r = fl + 1 if frac > Fraction(1, 2) else fl
            assert q[v, h] == max(-7, min(7, r)), (v, h, float(exact))
    assert near_tie < 3


def test_dequantisation_error_bound():
    """|q*s - W| <= s/2 wherever |W/s| <= 7.5 (up to the binary32 rounding
    of the quotient), and q = +-7 beyond."""
    rng = np.random.default_rng(2)
    w = f16(rng.normal(0, 0.1, size=(200, 128)))
    s = f16(rng.lognormal(-4, 0.7, size=128))
    q = rq.quantize(w, rq.F16, s).astype(np.float64)
    wv = w.view(np.float16).astype(np.float64)
    sv = s.view(np.float16).astype(np.float64)
    ratio = wv / sv
    inside = np.abs(ratio) <= 7.5 - 1e-6
    err = np.abs(q * sv - wv)
    assert np.all(err[inside] <= sv.repeat(200).reshape(128, 200).T[inside] * (0.5 + 1e-6))
    assert np.all(q[ratio > 7.5 + 1e-6] == 7) and np.all(q[ratio < -7.5 - 1e-6] == -7)


def test_round_trip_of_representable_weights():
    rng = np.random.default_rng(3)
    s = f16(rng.lognormal(-4, 0.5, size=96))
    qi = rng.integers(-7, 8, size=(50, 96)).astype(np.int8)
    w = f16(qi * s.view(np.float16).astype(np.float64))
    assert np.array_equal(rq.quantize(w, rq.F16, s), qi)


def test_pack_against_verify_oracle_unpack(oracle_mod):
    rng = np.random.default_rng(4)
    qi = rng.integers(-7, 8, size=(33, 64)).astype(np.int8)
    packed = rq.pack(qi)
    q2, nbad = oracle_mod.unpack(packed, 33, 64)
    assert nbad == 0 and np.array_equal(q2, qi)


def test_packed_head_through_verify_oracle(oracle_mod):
    """A one-hot hidden state with unit scales reads one quantised column of
    the packed head back out of the verify oracle's logits."""
    rng = np.random.default_rng(5)
    V, H = 40, 32
    w = f16(rng.normal(0, 0.2, size=(V, H)))
    acts = f16(rng.normal(0, 1.0, size=(10, H)))
    packed, s = rq.requantize(w, rq.F16, acts, rq.F16)
    q = rq.quantize(w, rq.F16, s)
    ones = f16([1.0] * H)
    for k in (0, 1, 17, 31):
        x = np.zeros(H)
        x[k] = 1.0
        lg = oracle_mod.logits(f16(x)[None, :], packed, ones, 1, V, H)
        assert np.array_equal(lg[0], q[:, k].astype(np.float32))


def test_calibration_amax_and_scales():
    rng = np.random.default_rng(6)
    a = rng.normal(0, 2.0, size=(7, 12))
    a16 = f16(a)
    am = rq.calib_amax(a16, rq.F16)
    vals = a16.view(np.float16).astype(np.float64)
    for h in range(12):
        assert am[h] == max(abs(vals[n, h]) for n in range(7))
    # bfloat16 patterns decode like torch's bfloat16
    bf = torch.tensor(a, dtype=torch.float32).to(torch.bfloat16)
    bits = bf.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(rq.decode(bits, rq.BF16), bf.float().numpy())
    am_bf = rq.calib_amax(bits, rq.BF16)
    assert np.array_equal(am_bf, bf.float().abs().max(dim=0).values.numpy())
    # s = amax / 7 stored in binary16: special values
    s = rq.scales_from_amax(np.array([7.0, 0.0, 1e-9, 65504.0 * 7, 3.5], np.float32))
    assert s.view(np.float16).tolist() == [1.0, 0.0, 0.0, 65504.0, 0.5]


def test_zero_and_infinite_scales_give_zero():
    w = f16([[1.0, -3.0, 0.25, 7.0]])
    s = np.array([0, 0x7C00, 0, 0x3C00], np.uint16)   # 0, +inf, 0, 1.0
    assert rq.quantize(w, rq.F16, s).tolist() == [[0, 0, 0, 7]]

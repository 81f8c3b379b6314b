"""The activation codes' split into three signed bytes, checked exhaustively
on the CPU.

The GPU paths turn a code |c| <= 0x7F7F7F into limbs (hi, mid, lo), each in
[-128, 127], with c = 2^16 hi + 2^8 mid + lo.  The staging kernels peel the
low byte off with sign extension; the fused staging instead reads the bytes
of the biased value c + 0x808080 and flips their top bit.  Both must give the
same (unique) signed-digit decomposition for every code in range."""
import numpy as np

CODE_MAX = 0x7F7F7F


def sext8(v):
    return ((v & 0xFF) ^ 0x80) - 0x80


def test_biased_bytes_equal_peeled_limbs_for_every_code():
    c = np.arange(-CODE_MAX, CODE_MAX + 1, dtype=np.int64)
    # peeled: low byte with sign extension, then the next
    lo = sext8(c)
    c1 = (c - lo) >> 8
    mid = sext8(c1)
    hi = (c1 - mid) >> 8
    # biased: bytes of c + 0x808080, top bit flipped, read as int8
    u = c + 0x808080
    assert u.min() >= 0 and u.max() < (1 << 24)
    b = [(((u >> (8 * i)) & 0xFF) ^ 0x80).astype(np.uint8).view(np.int8).astype(np.int64) for i in range(3)]
    assert np.array_equal(b[0], lo) and np.array_equal(b[1], mid) and np.array_equal(b[2], hi)
    for limb in (lo, mid, hi):
        assert limb.min() >= -128 and limb.max() <= 127
    assert np.array_equal((hi << 16) + (mid << 8) + lo, c)


def test_code_bound_is_the_largest_three_limb_value():
    # 0x7F7F7F is the largest code whose three limbs all stay below 128, and
    # -0x7F7F7F the most negative one used (the bound is symmetric)
    assert 127 * (1 << 16) + 127 * (1 << 8) + 127 == CODE_MAX
    assert -128 * (1 << 16) - 128 * (1 << 8) - 128 < -CODE_MAX

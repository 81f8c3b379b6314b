"""CPU oracle of the offline requantisation of the output head (calibrated
int4 lm_head).

TEST INFRASTRUCTURE ONLY: imported by the test suite and the CPU-baseline leg
of the benchmark, never by the GPU library or its binding.  Plain numpy in
binary32, following the definition step by step.

The step is the requantisation listing of "Qwen3.8-27B on a Single RTX 3090:
How Calibrated Quantization and Speculative Decoding Hit 1,000 tok/s",
Technical Insight: the per-hidden-channel scale is the largest absolute
activation of that channel over the calibration rows, divided by 7 (the int4
range used is [-7, 7]); each weight is divided by its channel's scale, rounded
to the nearest integer and clamped to [-7, 7].  "HyperQwen: 1,000 tok/s on a
Single RTX 3090 Through Aggressive Recurrent-State Speculation", Technical
Insight (lm_head paragraph), describes the same pipeline: activation ranges
on representative data, per-channel scales, 4-bit weights.

Readings where the pages leave the step open (each restated in the design
notes):
  * arithmetic is binary32: amax is exact, the division by 7 rounds once to
    binary32, and the stored scale is that value rounded to binary16 (the
    head format keeps fp16 scales);
  * the weight is divided by the stored binary16 scale (so that q * s is the
    dequantised weight the verify path uses), in binary32, rounded once;
  * rounding to an integer is round-half-to-even (torch.round), then the
    clamp to [-7, 7];
  * a channel whose stored scale is 0 (no activation, or amax / 7 below the
    binary16 range) quantises every weight to 0; an infinite scale also
    gives 0 (W / inf = 0);
  * weights and activations are binary16 or bfloat16 bit patterns and must
    be finite (a precondition).
The packed layout is the head format of the verify path: [V, H/2] bytes, the
even channel in the low nibble, the odd channel in the high nibble, two's
complement nibbles.
"""
from __future__ import annotations

import numpy as np

F16, BF16 = 0, 1


def decode(bits: np.ndarray, dtype: int) -> np.ndarray:
    """binary16 or bfloat16 bit patterns -> binary32 values (exact)."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    if dtype == F16:
        return bits.view(np.float16).astype(np.float32)
    if dtype == BF16:
        return (bits.astype(np.uint32) << 16).view(np.float32)
    raise ValueError(dtype)


def calib_amax(acts_bits: np.ndarray, dtype: int) -> np.ndarray:
    """Largest |activation| of each hidden channel over the calibration rows
    (acts [N, H]); binary32, exact."""
    a = decode(acts_bits, dtype)
    assert a.ndim == 2 and a.shape[0] >= 1
    assert np.all(np.isfinite(a)), "calibration activations must be finite"
    return np.max(np.abs(a), axis=0).astype(np.float32)


def scales_from_amax(amax: np.ndarray) -> np.ndarray:
    """s = amax / 7 in binary32, stored as binary16: returns the fp16 bit
    patterns [H]."""
    s32 = np.asarray(amax, np.float32) / np.float32(7.0)
    return s32.astype(np.float16).view(np.uint16)


def quantize(w_bits: np.ndarray, dtype: int, scales_bits: np.ndarray) -> np.ndarray:
    """q[v, h] = clamp(rne(W[v, h] / s[h]), -7, 7) as int8 [V, H]; 0 where
    s[h] is 0 or infinite."""
    w = decode(w_bits, dtype)
    assert np.all(np.isfinite(w)), "weights must be finite"
    s = np.ascontiguousarray(scales_bits, np.uint16).view(np.float16).astype(np.float32)
    assert not np.any(np.isnan(s)) and np.all(s >= 0), "scales must be >= 0"
    q = np.zeros(w.shape, np.int8)
    ok = (s > 0) & np.isfinite(s)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = w[:, ok] / s[ok]                      # binary32 division, one rounding
    q[:, ok] = np.clip(np.rint(ratio), -7, 7).astype(np.int8)   # half to even, clamp
    return q


def pack(q: np.ndarray) -> np.ndarray:
    """int8 [V, H] in [-7, 7] -> packed uint8 [V, H/2] (low nibble = even
    channel, high nibble = odd channel, two's complement)."""
    q = np.asarray(q, np.int8)
    V, H = q.shape
    assert H % 2 == 0
    lo = q[:, 0::2].astype(np.int16) & 0xF
    hi = q[:, 1::2].astype(np.int16) & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def requantize(w_bits: np.ndarray, w_dtype: int, acts_bits: np.ndarray, acts_dtype: int):
    """The whole offline step: (packed head [V, H/2], fp16 scale bits [H])."""
    s = scales_from_amax(calib_amax(acts_bits, acts_dtype))
    return pack(quantize(w_bits, w_dtype, s)), s

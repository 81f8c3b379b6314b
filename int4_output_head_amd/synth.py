"""Seeded synthetic inputs for the int4 verify path.

This module is shared by the oracle side and the GPU side of the tests and
the benchmark.  It draws random numbers and lays them out in the input
formats; it holds none of the method's arithmetic (no dequantisation, no dot
products, no argmax, no acceptance count).  Draft ids that must agree with
the target's greedy argmax are produced in two steps: ``draft_plan`` draws
the random parts, and ``finalize_drafts`` copies ids from an argmax that the
caller supplies (the oracle's, computed by the caller).

Workloads (no page gives tensors; all inputs are synthetic):

* shapes of a Qwen3.8-27B-class output head (vocabulary of about 152k rows,
  "HyperQwen: 1,000 tok/s on a Single RTX 3090 Through Aggressive
  Recurrent-State Speculation", Technical Insight, the section on the lm_head
  and on the draft vocabulary of 8192 tokens) with hidden size 5120;
* verify blocks of 7 drafted + up to 8 context-copied + 1 bonus positions
  ("HyperQwen on one RTX 3090: a first-time developer's guide to the
  381-token claim", "What actually became faster?"), T = 8 or 16;
* a batch of 64 requests x T = 4 (the 64-concurrent batch mode of the
  HyperQwen README, "The numbers behind that").

Random streams: the head (q, heavy rows, s) comes from one stream seeded by
``head_seed``; the hidden states of a trial from a second stream seeded by the
trial seed; the draft plan of a trial from a third.  numpy's PCG64 through a
SeedSequence of (tag, stream, seed).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

_TAG = 0x1A4  # fixed first word of every SeedSequence used here


def _rng(stream: int, seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([_TAG, stream, int(seed)])))


@dataclass(frozen=True)
class Config:
    name: str
    R: int          # independent requests sharing the head
    T: int          # verify positions per request
    V: int          # vocabulary rows
    H: int          # hidden size
    heavy_frac: float   # fraction of rows drawn from the heavy (+/-7) mixture
    draft: str      # draft recipe, see draft_plan
    p: float        # parameter of the draft recipe
    trials: int     # seeded trials (trial seeds 0 .. trials-1)
    desc: str

    @property
    def M(self) -> int:
        return self.R * self.T

    @property
    def weight_bytes(self) -> int:
        return self.V * self.H // 2


CONFIGS = {
    "tiny": Config("tiny", 1, 4, 4096, 256, 0.0, "fixed_prefix", 2, 1,
                   "tiny verify V=4096 H=256 T=4"),
    "draft_vocab": Config("draft_vocab", 1, 1, 8192, 5120, 0.0, "none", 0, 1000,
                          "draft-vocab head, single decode V=8192 H=5120 T=1"),
    "full_t8": Config("full_t8", 1, 8, 151936, 5120, 0.05, "geometric", 0.3, 20,
                      "full-vocab verify V=151936 H=5120 T=8"),
    "full_t16": Config("full_t16", 1, 16, 151936, 5120, 0.05, "bernoulli_all", 0.9, 20,
                       "full-vocab wide verify V=151936 H=5120 T=16"),
    "batch": Config("batch", 64, 4, 151936, 5120, 0.0, "geometric", 0.4, 5,
                    "batch verify 64 requests x T=4 V=151936 H=5120"),
    # two requests verified at once, each a wide verify block: 32 rows, the
    # smallest block past what one workgroup's registers hold
    "two_blocks_t16": Config("two_blocks_t16", 2, 16, 151936, 5120, 0.05, "bernoulli_all", 0.9, 10,
                             "two wide verify blocks (2 requests x T=16) V=151936 H=5120"),
    # one GPU's share of the full-vocabulary head split by vocabulary rows
    # over 8 GPUs (151936 / 8 = 18992 rows), at the wide verify block
    "shard_t16": Config("shard_t16", 1, 16, 18992, 5120, 0.05, "bernoulli_all", 0.9, 20,
                        "vocabulary shard of 8 (V=18992) wide verify H=5120 T=16"),
}


# ---------------------------------------------------------------- formats

def pack_int4(q: np.ndarray) -> np.ndarray:
    """Lay out int4 values [V, H] (int8 in [-7, 7]) as the canonical packed
    head [V, H/2] uint8: low nibble = even channel, high nibble = odd channel,
    two's-complement nibbles."""
    q = np.asarray(q, dtype=np.int8)
    V, H = q.shape
    assert H % 2 == 0
    u = q.view(np.uint8)
    return ((u[:, 0::2] & 0xF) | ((u[:, 1::2] & 0xF) << 4)).astype(np.uint8)


def f16_bits(a) -> np.ndarray:
    """float64 values -> binary16 bit patterns (round to nearest even)."""
    return np.asarray(a, dtype=np.float64).astype(np.float16).view(np.uint16)


# ---------------------------------------------------------------- head

def _uniform_q(rng, rows, H):
    return rng.integers(-7, 8, size=(rows, H), dtype=np.int8)


def _heavy_q(rng, rows, H):
    # Half of the values at +/-7 (uniform sign), the rest uniform in [-7, 7].
    at_edge = rng.random((rows, H)) < 0.5
    sign = np.where(rng.random((rows, H)) < 0.5, -7, 7).astype(np.int8)
    uni = rng.integers(-7, 8, size=(rows, H), dtype=np.int8)
    return np.where(at_edge, sign, uni).astype(np.int8)


def make_head(cfg: Config, head_seed: int = 0, keep_q: bool = False,
              chunk_rows: int = 4096) -> dict:
    """Packed head [V, H/2] uint8 and scales [H] (binary16 bits).

    Draw order: uniform q for all rows (in chunks of ``chunk_rows``), then the
    heavy rows (without replacement) and their values, then the scales
    ~ lognormal(mu=-4, sigma=0.5) rounded to binary16."""
    rng = _rng(0, head_seed)
    V, H = cfg.V, cfg.H
    packed = np.empty((V, H // 2), np.uint8)
    q_all = np.empty((V, H), np.int8) if keep_q else None
    for r0 in range(0, V, chunk_rows):
        r1 = min(V, r0 + chunk_rows)
        q = _uniform_q(rng, r1 - r0, H)
        packed[r0:r1] = pack_int4(q)
        if keep_q:
            q_all[r0:r1] = q
    n_heavy = int(round(cfg.heavy_frac * V))
    heavy = np.sort(rng.choice(V, size=n_heavy, replace=False)) if n_heavy else np.zeros(0, np.int64)
    if n_heavy:
        qh = _heavy_q(rng, n_heavy, H)
        packed[heavy] = pack_int4(qh)
        if keep_q:
            q_all[heavy] = qh
    scales = f16_bits(rng.lognormal(-4.0, 0.5, size=H))
    out = dict(packed=packed, scales=scales, heavy_rows=heavy)
    if keep_q:
        out["q"] = q_all
    return out


def make_hidden(cfg: Config, trial_seed: int) -> np.ndarray:
    """Hidden states [R*T, H] ~ N(0, 1) rounded to binary16 (bits)."""
    rng = _rng(1, trial_seed)
    return f16_bits(rng.standard_normal((cfg.M, cfg.H)))


# ---------------------------------------------------------------- drafts

def draft_plan(cfg: Config, trial_seed: int) -> dict:
    """Random part of the draft ids of one trial.

    Returns ``match`` [R, T-1] (positions that copy the target's argmax),
    ``must_differ`` [R, T-1] (the first position after the accepted prefix,
    whose id must differ from the argmax) and ``rand_ids`` [R, T-1] (ids used
    where ``match`` is false).  Recipes:

    fixed_prefix  positions < p copy the argmax, the rest are uniform ids
                  (no redraw: a random id may match by chance);
    geometric     accepted prefix k = min(geometric(p) - 1, T-1) per request;
                  position k differs from the argmax, later ones uniform;
    bernoulli_all with probability p all T-1 drafts match; otherwise one
                  position j ~ U{0..T-2} differs and all others match;
    none          T == 1, no drafts.
    """
    R, T, V = cfg.R, cfg.T, cfg.V
    n = T - 1
    rng = _rng(2, trial_seed)
    match = np.zeros((R, n), bool)
    must_differ = np.zeros((R, n), bool)
    rand_ids = rng.integers(0, V, size=(R, n), dtype=np.int64).astype(np.int32)
    if n == 0 or cfg.draft == "none":
        return dict(match=match, must_differ=must_differ, rand_ids=rand_ids)
    if cfg.draft == "fixed_prefix":
        k = min(int(cfg.p), n)
        match[:, :k] = True
    elif cfg.draft == "geometric":
        ks = np.minimum(rng.geometric(cfg.p, size=R) - 1, n)
        for i, k in enumerate(ks):
            match[i, :k] = True
            if k < n:
                must_differ[i, k] = True
    elif cfg.draft == "bernoulli_all":
        for i in range(R):
            if rng.random() < cfg.p:
                match[i, :] = True
            else:
                j = int(rng.integers(0, n))
                match[i, :] = True
                match[i, j] = False
                must_differ[i, j] = True
    else:
        raise ValueError(cfg.draft)
    return dict(match=match, must_differ=must_differ, rand_ids=rand_ids)


def finalize_drafts(cfg: Config, plan: dict, argmax_ids: np.ndarray) -> np.ndarray:
    """Draft ids [R, T-1] int32 from a plan and the target argmax [R*T]
    supplied by the caller.  A random id that must differ but equals the
    argmax is replaced by (id + 1) mod V."""
    R, T, V = cfg.R, cfg.T, cfg.V
    if T == 1:
        return np.zeros((R, 0), np.int32)
    am = np.asarray(argmax_ids, np.int64).reshape(R, T)[:, : T - 1]
    d = np.where(plan["match"], am, plan["rand_ids"].astype(np.int64))
    clash = plan["must_differ"] & (d == am)
    d = np.where(clash, (d + 1) % V, d)
    return d.astype(np.int32)


# ---------------------------------------------------------------- special inputs

def int_exact_inputs(M: int, V: int, H: int, seed: int) -> dict:
    """Inputs whose every partial sum is exactly representable in binary32:
    x integers in [-4, 4], s in {1, 1/2, 1/4}, q uniform in [-7, 7].  Every
    product is a multiple of 1/4 of magnitude <= 28, so with H <= 2^17 every
    partial sum is a multiple of 1/4 below 2^22 in magnitude: exact in any
    summation order."""
    rng = _rng(3, seed)
    q = _uniform_q(rng, V, H)
    x = rng.integers(-4, 5, size=(M, H)).astype(np.float64)
    s = rng.choice(np.array([1.0, 0.5, 0.25]), size=H)
    return dict(q=q, packed=pack_int4(q), hidden=f16_bits(x), scales=f16_bits(s))


def uniform_inputs(M: int, V: int, H: int, seed: int, heavy_frac: float = 0.0) -> dict:
    """Generic random inputs of any shape with the distributions above
    (q uniform in [-7, 7], s ~ lognormal(-4, 0.5), x ~ N(0, 1))."""
    rng = _rng(4, seed)
    q = _uniform_q(rng, V, H)
    n_heavy = int(round(heavy_frac * V))
    if n_heavy:
        rows = rng.choice(V, size=n_heavy, replace=False)
        q[rows] = _heavy_q(rng, n_heavy, H)
    s = f16_bits(rng.lognormal(-4.0, 0.5, size=H))
    x = f16_bits(rng.standard_normal((M, H)))
    return dict(q=q, packed=pack_int4(q), hidden=x, scales=s)


# ---------------------------------------------------------------- requantisation inputs

def bf16_bits(a) -> np.ndarray:
    """float64 values -> bfloat16 bit patterns (binary32 rounding to nearest
    even first, then the upper half rounded to nearest even)."""
    f = np.asarray(a, dtype=np.float64).astype(np.float32).view(np.uint32).astype(np.uint64)
    rounded = (f + 0x7FFF + ((f >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def requant_inputs(V: int, H: int, N: int, seed: int, w_dtype: str = "f16",
                   a_dtype: str = "f16") -> dict:
    """A synthetic full-precision head W [V, H] and N calibration rows of
    final hidden states [N, H], as bit patterns of ``w_dtype`` / ``a_dtype``
    ("f16" or "bf16").  No checkpoint or calibration set is available, so
    both are drawn: channel magnitudes c[h] ~ lognormal(0, 1) (a few channels
    carry much larger activations than the rest), activations N(0, 1) * c[h],
    weights N(0, 1) * 2 * c[h], so that weight / (largest activation / 7)
    spreads over about +-8 and a few per cent of the codes clamp."""
    rng = _rng(5, seed)
    c = rng.lognormal(0.0, 1.0, size=H)
    acts = rng.standard_normal((N, H)) * c
    W = np.empty((V, H), np.float64)
    for r0 in range(0, V, 8192):
        r1 = min(V, r0 + 8192)
        W[r0:r1] = rng.standard_normal((r1 - r0, H)) * (2.0 * c)
    enc = {"f16": f16_bits, "bf16": bf16_bits}
    return dict(W=enc[w_dtype](W), acts=enc[a_dtype](acts))

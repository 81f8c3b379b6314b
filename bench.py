"""Benchmark of the int4 lm_head verify path on one MI355X.

A step is one verify call: the whole path (activation codes, weight stream,
contraction, argmax, acceptance) over one block of synthetic hidden states,
with every input already resident in HBM.  The head is rotated over several
copies so that the 256 MB Infinity Cache cannot serve it.  Prints one JSON
line.

    python bench.py [--gpus 1] [--steps 200] [--warmup 20] [--config full_t16]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E peak, GB/s
INT8_PEAK_TOPS = 5000.0        # MI355X dense int8 MFMA peak, TOP/s
SINGLE_BLOCK_ROWS = 64         # larger blocks run the MFMA-bound batch kernels
SAMPLED_MAX_ROWS = 4096        # sampled calls: fused into the weight stream up to 64 rows, then
                               # the batch kernels' logits and a per-row selection
METRIC = "int4 lm_head verify: weight GB/s (% HBM peak) and verified tokens/s at T=16"
# what the path computes: int4 weights times 24-bit fixed-point activation
# codes (x*s, exact in binary32, rounded to 24 bits), run as three int8 MFMA
# limbs with exact integer sums, one rounding to binary32 per logit
DTYPE = "int4 x int24 (3 int8 MFMA limbs, exact integer sums, fp32 logits)"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def stored_argmax(name):
    path = os.path.join(ROOT, "tests", "golden", f"argmax_{name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        return json.load(f)


def host_threads():
    """Threads for the oracle on this host: the CPUs this process may run on,
    capped by OMP_NUM_THREADS (the host share of one GPU where it is set)."""
    n = len(os.sched_getaffinity(0))
    cap = os.environ.get("OMP_NUM_THREADS")
    if cap and cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, n)


def cpu_baseline(cfg, head, trials, n_threads, top_k=None, temperature=1.0, vmap=None, want_logits=False):
    """The oracle, as it is, on this host: whole verify steps of the same
    workload (bounded number of trials) -- the sampled oracle for top-k
    sampling, the draft-vocabulary oracle for a mapped head.  With
    want_logits the first trial's logits are returned too (the oracle writes
    them into the caller's array instead of a scratch one: the same work)."""
    from oracle import oracle, sampled, vocab_map
    from int4_output_head_amd import synth
    times = []
    first = None
    for trial in trials:
        x = synth.make_hidden(cfg, trial)
        drafts = np.zeros((cfg.R, cfg.T - 1), np.int32)
        t0 = time.perf_counter()
        if top_k is not None:
            ones = np.ones((cfg.R, cfg.T - 1))
            sampled.verify_sampled(x, head["packed"], head["scales"], drafts, ones, ones * 0.5, cfg.R,
                                   cfg.T, cfg.V, cfg.H, top_k, temperature, n_threads=n_threads)
        elif vmap is not None:
            vocab_map.verify_mapped(x, head["packed"], head["scales"], vmap, drafts, cfg.R, cfg.T,
                                    cfg.V, cfg.H, n_threads=n_threads)
        else:
            o = oracle.verify(x, head["packed"], head["scales"], drafts, cfg.R, cfg.T, cfg.V, cfg.H,
                              n_threads=n_threads, want_logits=want_logits and first is None)
            if first is None:
                first = o
        times.append(time.perf_counter() - t0)
    t = float(np.mean(times))
    res = dict(value=round(cfg.weight_bytes / t / 1e9, 4), unit="GB/s", cores=n_threads,
               kind="oracle", seconds_per_step=round(t, 6),
               verified_tok_s=round(cfg.M / t, 3),
               sample=f"{len(trials)} whole verify steps of the same workload (all {cfg.M} rows x "
                      f"{cfg.V} vocab rows), trial seeds {trials[0]}..{trials[-1]}, mean per step")
    return res, first


# HBM bytes per launch of the main kernel, from two rocprofv3 runs (FETCH_SIZE,
# then WRITE_SIZE) scaled by what the same counters read for a device copy of
# known size (factors 2.000 and 1.000); the summaries are in profiles/.  Each
# entry holds the SHA-256 of the kernel source it was measured on: once the
# source changes the entry no longer applies and `traffic` is null.
MEASURED_TRAFFIC = {
    "full_t16": dict(read=391_060_135, write=73_920, source="int4vh.hip",
                     source_sha256="578e0dc5ae34e588a913373167627327a2538b4141a10d5cb61fc0c3b60256ba"),
    "full_t8": dict(read=390_392_529, write=41_088, source="int4vh.hip",
                    source_sha256="578e0dc5ae34e588a913373167627327a2538b4141a10d5cb61fc0c3b60256ba"),
    "two_blocks_t16": dict(read=393_049_627, write=74_048, source="int4vh.hip",
                           source_sha256="578e0dc5ae34e588a913373167627327a2538b4141a10d5cb61fc0c3b60256ba"),
    "batch": dict(read=683_951_487, write=1_062_176, source="int4vh.hip",
                  source_sha256="578e0dc5ae34e588a913373167627327a2538b4141a10d5cb61fc0c3b60256ba"),
    "draft_vocab": dict(read=21_350_396, write=17_536, source="int4vh.hip",
                        source_sha256="578e0dc5ae34e588a913373167627327a2538b4141a10d5cb61fc0c3b60256ba"),
    "shard_t16": dict(read=50_761_953, write=74_944, source="int4vh.hip",
                      source_sha256="578e0dc5ae34e588a913373167627327a2538b4141a10d5cb61fc0c3b60256ba"),
    "full_t16_top16": dict(read=391_712_757, write=568_576, source="int4vh.hip",
                           source_sha256="578e0dc5ae34e588a913373167627327a2538b4141a10d5cb61fc0c3b60256ba"),
    "full_t16_top0": dict(read=391_481_381, write=358_912, source="int4vh.hip",
                          source_sha256="578e0dc5ae34e588a913373167627327a2538b4141a10d5cb61fc0c3b60256ba"),
    "two_blocks_t16_top16": dict(read=393_676_928, write=570_816, source="int4vh.hip",
                                 source_sha256="578e0dc5ae34e588a913373167627327a2538b4141a10d5cb61fc0c3b60256ba"),
    "batch_top16": dict(read=684_045_968, write=159_548_356, source="int4vh.hip",
                        source_sha256="578e0dc5ae34e588a913373167627327a2538b4141a10d5cb61fc0c3b60256ba"),
    "batch_top0": dict(read=684_042_427, write=156_644_640, source="int4vh.hip",
                       source_sha256="578e0dc5ae34e588a913373167627327a2538b4141a10d5cb61fc0c3b60256ba"),
    "requant": dict(read=1_555_894_656, write=388_956_160, source="requant.hip",
                    source_sha256="9626a04fb5fe559ea2d9ed02d060f37f8d35b7e5fb71bbd087b08539e02acfef"),
}


TRAFFIC_NOTE = ("HBM bytes per launch from rocprofv3 FETCH_SIZE and WRITE_SIZE runs of this exact kernel "
                "source (SHA-256 checked; summaries in profiles/), divided by this run's mean launch time")


def measured_traffic(key, t_launch):
    import hashlib
    rec = MEASURED_TRAFFIC.get(key)
    if rec is None:
        return None, None
    src = os.path.join(ROOT, "int4_output_head_amd", "csrc", rec["source"])
    with open(src, "rb") as f:
        if hashlib.sha256(f.read()).hexdigest() != rec["source_sha256"]:
            return None, None
    nbytes = rec["read"] + rec["write"]
    return round(nbytes / t_launch / 1e9, 2), nbytes


def roofline(cfg, t_launch, gbs, key=None):
    """Roofline of the dominant (main verify) kernel, t_launch being its mean
    duration by HIP events that take the kernel's own dispatch start and end.  Up to 16 rows the
    weight stream bounds it (algorithmic bytes V*H/2).  Beyond, the
    int8 MFMAs do: algorithmic work is one multiply-add per (row, vocabulary
    row, channel), 2*M*V*H int8 ops; the kernel executes three times that
    (three limbs per activation code), reported beside it."""
    traffic, traffic_bytes = measured_traffic(key or cfg.name, t_launch)
    note = TRAFFIC_NOTE if traffic is not None else "no counter run for this kernel source"
    if cfg.M <= SINGLE_BLOCK_ROWS:
        return {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                "traffic_bytes_per_launch": traffic_bytes, "traffic_source": note,
                "algorithmic_bytes_per_launch": cfg.weight_bytes}
    ops = 2.0 * cfg.M * cfg.V * cfg.H
    tops = ops / t_launch / 1e12
    return {"bound": "mfma", "achieved": round(tops, 2), "peak": INT8_PEAK_TOPS, "unit": "TOP/s",
            "frac": round(tops / INT8_PEAK_TOPS, 4), "traffic": traffic,
            "traffic_unit": "GB/s", "traffic_bytes_per_launch": traffic_bytes, "traffic_source": note,
            "algorithmic_ops_per_launch": ops,
            "executed_int8_tops": round(3 * tops, 2),
            "executed_frac": round(3 * tops / INT8_PEAK_TOPS, 4),
            "weight_gb_s": round(gbs, 2)}


CALIBRATION_COPY_BYTES = 388_956_160   # the packed full-vocabulary head


def calibration_copy(torch, dev):
    """Three device copies of a known number of bytes, to scale hardware byte
    counters (FETCH_SIZE / WRITE_SIZE) taken in the same process."""
    src = torch.empty(CALIBRATION_COPY_BYTES, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"calibration: 3 device copies of {CALIBRATION_COPY_BYTES} bytes")
    del src, dst


REQUANT = dict(V=151936, H=5120, N=4096)
# oracle trials of the CPU baseline per workload (about 10-30 s of CPU work)
CPU_TRIALS = {"tiny": 200, "draft_vocab": 100, "full_t8": 2, "full_t16": 2, "shard_t16": 8, "batch": 1,
              "two_blocks_t16": 1}


def bench_requant(args):
    """The offline requantisation of the full-vocabulary head (V=151936,
    H=5120, binary16 weights, 4096 binary16 calibration rows): one step is
    the whole tool (calibration maxima, scales, quantise + pack).  The pack
    kernel dominates; its roofline counts the bytes it must move: the
    binary16 head read once, the packed head written once, the scales."""
    import torch
    from int4_output_head_amd import binding, synth

    V, H, N = REQUANT["V"], REQUANT["H"], REQUANT["N"]
    dev = torch.device("cuda:0")
    binding.load_library()
    t0 = time.time()
    inp = synth.requant_inputs(V, H, N, seed=0)
    log(f"requant inputs generated in {time.time() - t0:.1f}s")
    W = torch.from_numpy(inp["W"].view(np.int16)).view(torch.float16).to(dev)
    acts = torch.from_numpy(inp["acts"].view(np.int16)).view(torch.float16).to(dev)
    stream = torch.cuda.current_stream(dev)
    if args.calibrate_copy:
        calibration_copy(torch, dev)

    # parity gate: scales and 256 sampled packed rows against the oracle
    from oracle import requant as rq
    packed, scales, _ = binding.requantize(W, acts)
    torch.cuda.synchronize()
    s_want = rq.scales_from_amax(rq.calib_amax(inp["acts"], rq.F16))
    rows = np.sort(np.random.default_rng(0).choice(V, 256, replace=False))
    got_rows = packed[torch.from_numpy(rows).to(dev)].cpu().numpy()
    gate = dict(scales_equal=bool(np.array_equal(scales.cpu().view(torch.int16).numpy().view(np.uint16),
                                                 s_want)),
                rows_checked=int(rows.size),
                rows_equal=int(np.sum(np.all(got_rows == rq.pack(rq.quantize(inp["W"][rows], rq.F16, s_want)),
                                              axis=1))))
    log(f"parity gate: {gate}")

    t_w = time.time()
    i = 0
    while i < args.warmup or time.time() - t_w < 0.5:
        binding.requantize(W, acts)
        i += 1
    torch.cuda.synchronize()
    steps = args.steps
    k0 = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    k1 = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    b0 = torch.cuda.Event(enable_timing=True)
    b1 = torch.cuda.Event(enable_timing=True)
    amax = torch.empty(H, dtype=torch.float32, device=dev)
    # whole steps back to back (no per-call events: a timed launch costs the
    # host more than a plain one), then the pack kernel alone by events on
    # its own dispatch
    b0.record(stream)
    for i in range(steps):
        binding.requant_amax(acts, amax)
        sc = binding.requant_scales(amax)
        binding.requant_pack(W, sc)
    b1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = b0.elapsed_time(b1) / steps
    for i in range(steps):
        binding.requant_pack(W, sc, events=(k0[i], k1[i]))
    torch.cuda.synchronize()
    per_k = np.array([a.elapsed_time(b) for a, b in zip(k0, k1)])
    t_launch = float(per_k.mean()) * 1e-3
    pack_bytes = V * H * 2 + V * H // 2 + H * 2
    step_bytes = pack_bytes + N * H * 2
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = pack_bytes / t_launch / 1e9
    result = {
        "metric": "int4 lm_head requantisation: HBM GB/s of the whole offline step",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"requantise + pack the full-vocab head V={V} H={H} binary16 "
                               f"with {N} binary16 calibration rows",
                   "V": V, "H": H, "N": N, "timing": "eager, HIP events around the whole step"},
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "pack_kernel_us": {"mean": round(per_k.mean() * 1e3, 3),
                           "p10": round(np.percentile(per_k, 10) * 1e3, 3),
                           "p50": round(np.percentile(per_k, 50) * 1e3, 3),
                           "p90": round(np.percentile(per_k, 90) * 1e3, 3)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic("requant", t_launch)[0],
                     "traffic_bytes_per_launch": measured_traffic("requant", t_launch)[1],
                     "algorithmic_bytes_per_launch": pack_bytes},
        "parity_gate": gate,
    }
    if not args.no_cpu_baseline:
        n_rows = 8192
        t0 = time.time()
        s16 = rq.scales_from_amax(rq.calib_amax(inp["acts"], rq.F16))
        rq.pack(rq.quantize(inp["W"][:n_rows], rq.F16, s16))
        t = time.time() - t0
        nbytes = n_rows * H * 2 + n_rows * H // 2 + H * 2 + N * H * 2
        result["cpu_baseline"] = {
            "value": round(nbytes / t / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "seconds": round(t, 3),
            "sample": f"the oracle's calibration maxima over all {N} rows, scales, and "
                      f"quantise + pack of the first {n_rows} of {V} head rows (numpy, one thread)"}
    print(json.dumps(result), flush=True)


def bench_stream(args):
    """The reference line for the weight stream: a plain read-only pass over a
    buffer of the packed full-vocabulary head's size (388,956,160 B), with
    two copies rotated so the 256 MB Infinity Cache cannot serve it; mode 0
    loads into registers, mode 1 copies into LDS with the verify kernel's
    instruction.  One step is one pass."""
    import torch
    from int4_output_head_amd import binding

    dev = torch.device("cuda:0")
    binding.load_library()
    nbytes = CALIBRATION_COPY_BYTES
    gen = torch.Generator(device=dev).manual_seed(0)
    bufs = [torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), dtype=torch.int32, device=dev, generator=gen)
            for _ in range(2)]
    # the kernel reads every byte: the xor of its per-wave words is the xor
    # of the buffer's 32-bit words (computed on the host)
    out = binding.stream_read(bufs[0], 0)
    torch.cuda.synchronize()
    want = int(np.bitwise_xor.reduce(bufs[0].cpu().numpy().view(np.uint32)))
    got = int(np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32)))
    res = {}
    for mode in (0, 1):
        for i in range(max(args.warmup, 20)):
            binding.stream_read(bufs[i % 2], mode, out=out)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
        for i in range(args.steps):
            binding.stream_read(bufs[i % 2], mode, out=out, events=ev[i])
        torch.cuda.synchronize()
        per = np.array([a.elapsed_time(b) for a, b in ev]) * 1e-3
        res[mode] = dict(us_mean=round(float(per.mean()) * 1e6, 3),
                         us_p10=round(float(np.percentile(per, 10)) * 1e6, 3),
                         us_p90=round(float(np.percentile(per, 90)) * 1e6, 3),
                         GB_s=round(nbytes / float(per.mean()) / 1e9, 2))
        log(f"stream mode {mode}: {res[mode]}")
    best = max(res.values(), key=lambda r: r["GB_s"])
    result = {
        "metric": "read-only HBM stream of a head-sized buffer: GB/s (the weight stream's reference line)",
        "value": best["GB_s"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(best["us_mean"] / 1e3, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "u8 (read only)", "data": "synthetic",
        "config": {"workload": f"read {nbytes} B once per step, 2 buffers rotated",
                   "bytes": nbytes, "timing": "eager, HIP events on each kernel's own dispatch"},
        "modes": {"registers (global_load_dwordx4)": res[0], "lds (global_load_lds_dwordx4)": res[1]},
        "roofline": {"bound": "hbm", "achieved": best["GB_s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(best["GB_s"] / HBM_PEAK_GBS, 4), "traffic": None,
                     "algorithmic_bytes_per_launch": nbytes},
        "parity_gate": {"xor_of_buffer_equal": got == want},
        "cpu_baseline": None,
        "cpu_baseline_note": "a measurement kernel with no oracle counterpart",
    }
    print(json.dumps(result), flush=True)


SWEEP_ROWS = (1, 2, 4, 8, 16, 17, 20, 24, 28, 32, 40, 48, 56, 64, 96, 128, 192, 256, 512)


def bench_sweep(args):
    """Cost of one verify call against the number of rows M it verifies (M
    requests of one position each: the weight-stream path up to 16 rows,
    token groups of 16 up to 64, the matrix-core batch path beyond),
    full-vocabulary head V=151936, H=5120, two head copies rotated.  Per M: the whole call in a HIP graph of 20 calls
    (replayed after an untimed warm-up) and the main kernel alone (HIP events,
    eager).  The leg's value is the verified rows/s at M = 32 (with
    --sweep-rows not naming 32: at the largest M named)."""
    import torch
    from int4_output_head_amd import binding, synth

    dev = torch.device("cuda:0")
    binding.load_library()
    cfg = synth.CONFIGS["full_t16"]
    head = synth.make_head(cfg)
    w0 = torch.from_numpy(head["packed"]).to(dev)
    ws = [w0, w0.clone()]
    s = torch.from_numpy(head["scales"]).view(torch.float16).to(dev)
    rows = args.sweep_rows or SWEEP_ROWS
    rows_max = max(rows)
    rng = np.random.default_rng(0)
    x_all = torch.from_numpy(synth.f16_bits(rng.standard_normal((rows_max, cfg.H)))).view(torch.float16).to(dev)
    stream = torch.cuda.current_stream(dev)
    if args.calibrate_copy:
        calibration_copy(torch, dev)
    curve = []
    for M in rows:
        x = x_all[:M].reshape(M, 1, cfg.H).contiguous()
        work = binding.Workspace(binding.workspace_bytes(M, 1, cfg.V, cfg.H), dev)
        for i in range(10):
            binding.verify_batch(x, ws[i % 2], s, None, workspace=work)
        torch.cuda.synchronize()
        n_ev = 40
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_ev)]
        for i in range(n_ev):
            binding.verify_batch(x, ws[i % 2], s, None, workspace=work, events=ev[i])
        torch.cuda.synchronize()
        main_us = float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e3
        cap = torch.cuda.Stream(dev)
        cap.wait_stream(stream)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(cap):
            binding.verify_batch(x, ws[0], s, None, workspace=work)
            torch.cuda.synchronize()
            with torch.cuda.graph(g, stream=cap):
                for i in range(20):
                    binding.verify_batch(x, ws[i % 2], s, None, workspace=work)
        torch.cuda.synchronize()
        t_w = time.time()
        while time.time() - t_w < 0.2:
            g.replay()
            torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 5
        g0.record(stream)
        for _ in range(reps):
            g.replay()
        g1.record(stream)
        torch.cuda.synchronize()
        us = g0.elapsed_time(g1) * 1e3 / (reps * 20)
        rec = dict(M=M, us_per_call=round(us, 2), main_kernel_us=round(main_us, 2),
                   weight_GB_s=round(cfg.weight_bytes / (us * 1e-6) / 1e9, 1),
                   rows_per_s=round(M / (us * 1e-6), 1),
                   int8_TOPs_algorithmic=round(2.0 * M * cfg.V * cfg.H / (main_us * 1e-6) / 1e12, 1))
        curve.append(rec)
        log(f"sweep {rec}")
        del work, g
    at = {r["M"]: r for r in curve}
    m_val = 32 if 32 in at else max(at)
    result = {
        "metric": "int4 lm_head verify: verified rows/s against rows per call (full vocabulary)",
        "value": at[m_val]["rows_per_s"], "unit": "rows/s", "n_gpus": 1, "steps": 100, "warmup": 10,
        "ms_per_step": round(at[m_val]["us_per_call"] / 1e3, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": DTYPE, "data": "synthetic",
        "config": {"workload": "verify calls of M rows, V=151936 H=5120, M in " + str(list(rows)),
                   "value_at_rows": m_val,
                   "timing": "HIP graph of 20 calls replayed 5x per M; main kernel by HIP events"},
        "curve": curve,
        "ratio_32_to_16_rows": (round(at[32]["us_per_call"] / at[16]["us_per_call"], 3)
                                if 32 in at and 16 in at else None),
        "cpu_baseline": None,
        "cpu_baseline_note": "the oracle's cost grows linearly with M; see the full_t16 and batch legs",
    }
    print(json.dumps(result), flush=True)


def bench_context_copy(args):
    """The context-copy drafter on the workload of the wide verify block: a
    25,000-token synthetic prompt per request, a 16-token key whose tail
    quotes the prompt, 8 proposed tokens (verify positions 7-14).  One step
    is one drafter call; timed for 1 request (value) and for 64."""
    import torch
    from int4_output_head_amd import binding

    dev = torch.device("cuda:0")
    binding.load_library()
    from oracle import context_copy as cc
    L, n_max, n_out = 25000, 16, 8
    res = {}
    for R in (1, 64):
        rng = np.random.default_rng(R)
        prompts = rng.integers(0, 151936, size=(R, L)).astype(np.int32)
        keys = np.empty((R, n_max), np.int32)
        for r in range(R):
            s0 = int(rng.integers(n_max, L - n_out))
            keys[r] = prompts[r, s0 - n_max:s0]
        pr = torch.from_numpy(prompts.reshape(-1)).to(dev)
        offs = torch.from_numpy(np.arange(R + 1, dtype=np.int64) * L).to(dev)
        kt = torch.from_numpy(keys).to(dev)
        tok, cnt, end, ln = binding.context_copy(pr, offs, kt, n_min=2, n_out=n_out)
        torch.cuda.synchronize()
        ok = 0
        for r in range(min(R, 8)):
            o = cc.propose(prompts[r], keys[r], 2, n_out)
            ok += int(o["match_end"] == int(end[r]) and tok[r, : o["count"]].cpu().tolist() == o["tokens"].tolist())
        for _ in range(max(args.warmup, 50)):
            binding.context_copy(pr, offs, kt, n_min=2, n_out=n_out)
        torch.cuda.synchronize()
        # whole calls back to back (no per-call events: a timed launch costs
        # the host more than a plain one), then the kernel alone by events
        # on its own dispatch
        b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        b0.record()
        for i in range(args.steps):
            binding.context_copy(pr, offs, kt, n_min=2, n_out=n_out)
        b1.record()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
        for i in range(args.steps):
            binding.context_copy(pr, offs, kt, n_min=2, n_out=n_out, events=ev[i])
        torch.cuda.synchronize()
        per = np.array([a.elapsed_time(b) for a, b in ev]) * 1e3
        res[R] = dict(us_per_call=round(b0.elapsed_time(b1) * 1e3 / args.steps, 3),
                      kernel_us=round(float(per.mean()), 3), parity_checked=min(R, 8), parity_equal=ok)
        log(f"context copy R={R}: {res[R]}")
    t1 = res[1]["kernel_us"] * 1e-6
    nbytes = L * 4 + n_max * 4 + n_out * 4
    gbs = nbytes / t1 / 1e9
    t0 = time.perf_counter()
    rng = np.random.default_rng(5)
    p = rng.integers(0, 151936, size=L)
    n_cpu = 20
    for _ in range(n_cpu):
        cc.propose(p, p[1000:1016], 2, n_out)
    t_cpu = (time.perf_counter() - t0) / n_cpu
    result = {
        "metric": "context-copy drafter: proposals per second (8 tokens from a 25k-token prompt)",
        "value": round(1.0 / (res[1]["us_per_call"] * 1e-6), 1), "unit": "proposals/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(res[1]["us_per_call"] / 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "i32",
        "data": "synthetic",
        "config": {"workload": f"prompt lookup over a {L}-token prompt, key {n_max}, {n_out} proposed",
                   "L": L, "n_max": n_max, "n_out": n_out, "timing": "eager, HIP events"},
        "batch_64_requests": {"us_per_call": res[64]["us_per_call"], "kernel_us": res[64]["kernel_us"],
                              "proposals_per_s": round(64 / (res[64]["us_per_call"] * 1e-6), 1)},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 3), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 6), "traffic": None,
                     "algorithmic_bytes_per_launch": nbytes,
                     "note": "one request reads 100 KB: launch and latency bound"},
        "parity_gate": {R: {"checked": v["parity_checked"], "equal": v["parity_equal"]} for R, v in res.items()},
        "cpu_baseline": {"value": round(1.0 / t_cpu, 2), "unit": "proposals/s", "cores": 1, "kind": "oracle",
                         "sample": f"{n_cpu} oracle proposals over one {L}-token prompt (numpy, one thread)"},
    }
    print(json.dumps(result), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="full_t16")
    ap.add_argument("--copies", type=int, default=0, help="head copies to rotate (0: auto)")
    ap.add_argument("--cpu-trials", type=int, default=0, help="oracle trials of the CPU baseline (0: per workload)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--top-k", type=int, default=0,
                    help="sampled verification: top-k sampling with this k (0: greedy)")
    ap.add_argument("--temperature", type=float, default=1.0)
    ap.add_argument("--full-softmax", action="store_true",
                    help="sampled verification over the whole vocabulary (top_k = 0)")
    ap.add_argument("--sweep-rows", default="",
                    help="--config sweep: comma-separated row counts (default: the whole curve)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run a plain device copy of head-sized buffers (a known "
                         "number of bytes) to scale hardware byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path runs on a single MI355X; see the sharding notes)", file=sys.stderr)
        sys.exit(2)
    if args.sweep_rows:
        try:
            args.sweep_rows = tuple(int(m) for m in args.sweep_rows.split(","))
        except ValueError:
            args.sweep_rows = ()
        if not args.sweep_rows or min(args.sweep_rows) < 1 or max(args.sweep_rows) > 4096:
            print("--sweep-rows: comma-separated row counts from 1 to 4096", file=sys.stderr)
            sys.exit(2)

    if args.config == "requant":
        bench_requant(args)
        return
    if args.config == "context_copy":
        bench_context_copy(args)
        return
    if args.config == "stream":
        bench_stream(args)
        return
    if args.config == "sweep":
        bench_sweep(args)
        return

    import torch
    from int4_output_head_amd import binding, synth

    cfg = synth.CONFIGS[args.config]
    dev = torch.device("cuda:0")
    binding.load_library()
    props = torch.cuda.get_device_properties(dev)
    log(f"device {props.name} CUs {props.multi_processor_count}; config {cfg.desc}")

    t0 = time.time()
    head = synth.make_head(cfg)
    log(f"head generated in {time.time() - t0:.1f}s")
    if args.copies:
        copies = args.copies
    elif cfg.weight_bytes < 4 << 20:
        copies = 1        # fits one XCD's L2: the call is dispatch-bound, rotation cannot change that
    else:
        copies = max(2, -(-600_000_000 // cfg.weight_bytes))  # > 256 MB MALL
    w0 = torch.from_numpy(head["packed"]).to(dev)
    ws = [w0] + [w0.clone() for _ in range(copies - 1)]
    s = torch.from_numpy(head["scales"]).view(torch.float16).to(dev)

    stored = stored_argmax(cfg.name)
    n_trials = min(cfg.trials, 20)
    xs, ds, ref_ids = [], [], []
    for trial in range(n_trials):
        x = synth.make_hidden(cfg, trial)
        xs.append(torch.from_numpy(x).view(torch.float16).to(dev).reshape(cfg.R, cfg.T, cfg.H))
        ids = None
        if stored is not None and str(trial) in stored["trials"]:
            ids = np.array(stored["trials"][str(trial)]["argmax"], np.int32)
        ref_ids.append(ids)
        if cfg.T > 1:
            base = ids if ids is not None else np.zeros(cfg.M, np.int32)
            d = synth.finalize_drafts(cfg, synth.draft_plan(cfg, trial), base)
            ds.append(torch.from_numpy(d).to(dev))
        else:
            ds.append(None)
    if stored is None:
        log("no stored oracle argmax for this config: drafts are not aligned with the target")

    if args.calibrate_copy:
        calibration_copy(torch, dev)

    # (a sampled call above 64 rows also keeps its logits in the workspace)
    ws_size = binding.sampled_workspace_bytes if (args.top_k > 0 or args.full_softmax) else binding.workspace_bytes
    work = binding.Workspace(ws_size(cfg.R, cfg.T, cfg.V, cfg.H), dev)
    stream = torch.cuda.current_stream(dev)

    # The draft-vocabulary head: its rows are a subset of the full vocabulary
    # (a sorted random subset of 151936 token ids), and the step reports
    # token ids through the row -> token map.
    vmap_np = None
    if cfg.name == "draft_vocab":
        vmap_np = np.sort(np.random.default_rng(0).choice(151936, cfg.V, replace=False)).astype(np.int32)
        vmap = torch.from_numpy(vmap_np).to(dev)

    # Sampled verification (top-k sampling at a temperature): drafter
    # probabilities U(0.5, 1) for the 7 model-drafted positions, 1 for the
    # positions copied from the context, and seeded uniforms.
    sampled = args.top_k > 0 or args.full_softmax
    if sampled and cfg.M > SAMPLED_MAX_ROWS:
        raise SystemExit(f"--top-k / --full-softmax need at most {SAMPLED_MAX_ROWS} rows per call")
    qs, us = [], []
    if sampled and cfg.T > 1:
        for trial in range(n_trials):
            rng = np.random.default_rng(1000 + trial)
            q = np.ones((cfg.R, cfg.T - 1), np.float32)
            q[:, :7] = rng.uniform(0.5, 1.0, size=(cfg.R, min(7, cfg.T - 1)))
            qs.append(torch.from_numpy(q).to(dev))
            us.append(torch.from_numpy(rng.random((cfg.R, cfg.T - 1)).astype(np.float32)).to(dev))

    def nacc_of(out):
        return out[5] if sampled else out[2]

    def step(i, events=None):
        if sampled:
            q = qs[i % n_trials] if qs else None
            u = us[i % n_trials] if us else None
            return binding.verify_sampled(xs[i % n_trials], ws[i % copies], s, ds[i % n_trials], q, u,
                                          top_k=args.top_k, temperature=args.temperature,
                                          workspace=work, events=events)
        if events is not None:
            return binding.verify_batch(xs[i % n_trials], ws[i % copies], s, ds[i % n_trials],
                                        workspace=work, events=events)
        if vmap_np is not None:
            return binding.verify_mapped(xs[i % n_trials], ws[i % copies], s, vmap, ds[i % n_trials],
                                         workspace=work)
        return binding.verify_batch(xs[i % n_trials], ws[i % copies], s, ds[i % n_trials],
                                    workspace=work)

    # parity gate against the stored oracle argmax (ids may differ only at near ties)
    gate = dict(rows=0, ids_equal=0, near_tie_rows_allowed=0)
    for trial in range(n_trials):
        out = step(trial)
        amax = out[1]
        if ref_ids[trial] is not None:
            g = amax.cpu().numpy()
            if vmap_np is not None:
                g = np.searchsorted(vmap_np, g)          # token ids back to head rows
            gate["rows"] += cfg.M
            gate["ids_equal"] += int(np.sum(g == ref_ids[trial]))
            gaps = np.array(stored["trials"][str(trial)]["gap"])
            am = np.array(stored["trials"][str(trial)]["amax"])
            gate["near_tie_rows_allowed"] += int(np.sum(gaps < 2e-3 * am))
    torch.cuda.synchronize()
    log(f"parity gate vs stored oracle argmax: {gate}")

    # warm-up: at least --warmup calls and at least half a second of work (the
    # first calls after start read low until clocks settle)
    t_w = time.time()
    i = 0
    while i < args.warmup or time.time() - t_w < 0.5:
        step(i)
        i += 1
        if i % 50 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    log(f"warm-up: {i} calls")

    # (1) eager launches with HIP events: around each whole call (staging
    #     kernel + main kernel) and, through the instrumented entry point, on
    #     the main kernel's own dispatch (its start and end timestamps) --
    #     the dominant kernel whose duration the roofline uses
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    k0 = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    k1 = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    t_begin = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_begin.record(stream)
    for i in range(args.steps):
        starts[i].record(stream)
        step(i, events=(k0[i], k1[i]))
        ends[i].record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    eager_ms = t_begin.elapsed_time(t_end) / args.steps
    per = np.array([a.elapsed_time(b) for a, b in zip(starts, ends)])  # ms per call
    per_k = np.array([a.elapsed_time(b) for a, b in zip(k0, k1)])      # ms per main kernel

    # (2) the steps captured in a HIP graph and replayed (how a serving loop
    #     issues verify steps): whole-job throughput
    calls_per_graph = min(args.steps, 20)
    replays = max(1, args.steps // calls_per_graph)
    cap = torch.cuda.Stream(dev)
    cap.wait_stream(stream)
    outs = []
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cap):
        step(0)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=cap):
            for i in range(calls_per_graph):
                outs.append(step(i))
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    # every output of the replay equals the eager result of the same step
    replay_ok = True
    for i in (0, calls_per_graph - 1):
        ref = step(i)
        torch.cuda.synchronize()
        replay_ok &= all((a is None and b is None) or torch.equal(a, b) for a, b in zip(ref, outs[i]))
    # untimed replays first: the first few milliseconds after a capture run
    # slow (about 10% per step here), as after any change of launch pattern
    t_w = time.time()
    n_warm = 0
    while n_warm < 5 or time.time() - t_w < 0.3:
        graph.replay()
        n_warm += 1
        if n_warm % 10 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    g0 = torch.cuda.Event(enable_timing=True)
    g1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    g0.record(stream)
    for _ in range(replays):
        graph.replay()
    g1.record(stream)
    torch.cuda.synchronize()
    graph_steps = replays * calls_per_graph
    ms_per_step = g0.elapsed_time(g1) / graph_steps
    committed_tokens = sum(int(nacc_of(o).to(torch.int64).sum().item()) + cfg.R for o in outs) * replays

    t_launch = float(per_k.mean()) * 1e-3
    wbytes = cfg.weight_bytes
    value = wbytes / (ms_per_step * 1e-3) / 1e9
    achieved = wbytes / t_launch / 1e9
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": graph_steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE,
        "data": "synthetic",
        "config": {"workload": cfg.desc, "V": cfg.V, "H": cfg.H, "R": cfg.R, "T": cfg.T,
                   "head_copies_rotated": copies, "trials": n_trials,
                   **({"vocab_map": f"rows map to a sorted random {cfg.V} of 151936 token ids"}
                      if vmap_np is not None else {}),
                   **({"sampling": (f"top-{args.top_k}" if args.top_k else "whole vocabulary")
                                    + f" at temperature {args.temperature}"}
                      if sampled else {}),
                   "timing": f"HIP graph of {calls_per_graph} steps replayed {replays}x "
                             f"after {n_warm} untimed replays"},
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "verified_tok_s": round(cfg.M / (ms_per_step * 1e-3), 1),
        "committed_tok_s": round(committed_tokens / (graph_steps * ms_per_step * 1e-3), 1),
        "eager": {"ms_per_step": round(eager_ms, 5),
                  "GB_s": round(wbytes / (eager_ms * 1e-3) / 1e9, 2)},
        "call_us": {"mean": round(per.mean() * 1e3, 3), "p10": round(np.percentile(per, 10) * 1e3, 3),
                    "p50": round(np.percentile(per, 50) * 1e3, 3),
                    "p90": round(np.percentile(per, 90) * 1e3, 3)},
        "main_kernel_us": {"mean": round(per_k.mean() * 1e3, 3),
                           "p10": round(np.percentile(per_k, 10) * 1e3, 3),
                           "p50": round(np.percentile(per_k, 50) * 1e3, 3),
                           "p90": round(np.percentile(per_k, 90) * 1e3, 3)},
        "roofline": roofline(cfg, t_launch, achieved,
                             key=f"{cfg.name}_top{args.top_k}" if sampled else cfg.name),
        "graph_replay_matches_eager": bool(replay_ok),
        "parity_gate": gate,
    }
    if not args.no_cpu_baseline:
        n_threads = host_threads()
        n_cpu = args.cpu_trials or CPU_TRIALS.get(cfg.name, 2)
        log(f"cpu baseline: oracle on {n_threads} threads, {n_cpu} trials")
        plain = not sampled and vmap_np is None
        cb, first = cpu_baseline(cfg, head, list(range(n_cpu)), n_threads,
                                 top_k=args.top_k if sampled else None, temperature=args.temperature,
                                 vmap=vmap_np, want_logits=plain)
        cb["cpu_count"] = os.cpu_count()
        cb["affinity_cpus"] = len(os.sched_getaffinity(0))
        cb["omp_num_threads"] = os.environ.get("OMP_NUM_THREADS")
        if cfg.name in ("tiny", "draft_vocab"):
            st, _ = cpu_baseline(cfg, head, list(range(n_cpu)), 1, vmap=vmap_np)
            cb["single_thread"] = {k: st[k] for k in ("value", "unit", "cores", "seconds_per_step",
                                                      "verified_tok_s", "sample")}
        result["cpu_baseline"] = cb
        if plain and first is not None and "logits" in first:
            # the GPU's outputs and logits of trial 0 against the oracle's,
            # element by element (the oracle ran with zero drafts: its
            # acceptance count is recomputed for trial 0's drafts)
            from tests import parity
            d0 = ds[0].cpu().numpy() if ds[0] is not None else None
            lmax0, ids0, nacc0, lg0 = binding.verify_batch(xs[0], ws[0], s, ds[0], logits=True, workspace=work)
            torch.cuda.synchronize()
            g = dict(logits_max=lmax0.cpu().numpy(), argmax_ids=ids0.cpu().numpy(),
                     n_accepted=nacc0.cpu().numpy(), logits=lg0.cpu().numpy())
            o0 = dict(first)
            o0["n_accepted"] = parity.accept_from(o0["argmax_ids"], d0, cfg.R, cfg.T)
            result["parity_gate"]["logits_trial0"] = parity.check(g, o0, cfg.R, cfg.T, d0)
            log(f"trial 0 logits against the oracle: {result['parity_gate']['logits_trial0']}")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

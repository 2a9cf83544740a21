#!/usr/bin/env python3
"""Benchmark: KATA causal forward throughput on one MI355X.

One step = one kata_forward call over the whole long-context workload
(B=1, H=16, T=131072, d=dv=64, bf16 q/k/v, fp32 P, chunk 64 by default): the
chunk-state kernel, the associative scan of the leaf states with the final-state
export, and the intra-chunk kernel (projection, packed PSD features, prefix
readout, masked squared score tile, output gate).  Inputs are seeded synthetic
tensors already resident in HBM; the timed region covers exactly K steps
bracketed by device synchronisations.

Consecutive steps take different input batches (N distinct seeded batches, cycled),
so no step finds its inputs in the 256 MB last-level cache because the step before
read the same tensors.  Before the W warmup steps the step runs untimed for a short
settle period: an idle MI355X needs on the order of 100 ms of load before its clocks
reach their working level, and a handful of warmup steps (a few ms) is not enough.

Prints ONE JSON line with the metric, a roofline entry for the dominant kernel
(its duration measured live with HIP events recorded by the library on the
stream it launches on) and the CPU oracle timed on a bounded sample of the same
workload on the host's cores.  In the K timed steps only the dominant kernel's launch
stamps events (each stamping launch adds a few microseconds of dispatch gap); the
per-kernel breakdown comes from a pass of K steps before them in which every launch
stamps one.

    python bench.py [--steps K] [--warmup W] [--chunk C] [--no-cpu-baseline]
    python bench.py --decode     # the recurrent decode step instead (its own JSON line)
    python bench.py --flash      # the flash-style O(T^2) forward on the 340M-layer workload
    python bench.py --backward   # the chunked-state backward on the long-context workload
    python bench.py --decay      # the decay-gated forward on the long-context workload
    python bench.py --decode --delta   # the DeltaKATA decode step (prefill by its recurrent forward)
    python bench.py --decode --packed  # the decode step on the packed symmetric state (136 rows)
    python bench.py --delta      # the DeltaKATA forward, chunked form, on the long-context workload
    python bench.py --factors 2  # KATA-M2 (two concatenated PSD factors) on the long-context workload
    python bench.py --workload mid     # the forward on the mid workload (B=4 H=8 T=4096), warm and flushed
    python bench.py --workload lm340m  # the forward on the 340M-layer workload (B=8 H=16 T=2048)
    python bench.py --stream-probe     # torch's streaming kernels (read, copy, 3:1) for the practical ceilings
    python bench.py --copy-calibration MIB  # plain device copies (counter calibration; scan-sized copies)

The decode mode prefills 256 streams x 16 heads with 8192 tokens (kata_forward with
the final-state export), then times 1024 kata_decode_step calls, each of which reads
and writes the 272.6 MB fp32 state once.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KATA causal fwd tokens/sec at T=131072 + % of MFMA/HBM peak (1 GPU)"
MG_METRIC = ("KATA-M{g} (g={g} concatenated PSD factors) causal fwd tokens/sec at T=131072 "
             "+ % of HBM peak (1 GPU)")
SG_METRIC = ("KATA-Sigma{g} (g={g} summed PSD factors) causal fwd tokens/sec at T=131072 "
             "+ % of HBM peak (1 GPU)")
DECAY_METRIC = "KATA decay-gated causal fwd tokens/sec at T=131072 + % of HBM peak (1 GPU)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 MFMA
KERNELS = ("kata_chunk_state", "kata_state_scan", "kata_chunk_intra")


def time_steps(torch, step, stream, steps, n_events, stamp, every=1):
    """Run exactly `steps` calls step(i, events) on `stream` between two device
    synchronisations.  Only the events at the indices in `stamp` reach the launches (the
    rest are None), and only on the steps i with i % every == 0: each launch that stamps an
    event costs a few microseconds of dispatch gap (on the long forward, stamping the
    intra launch's start and end on every step measured 0.342 ms per step against 0.331 ms
    with no stamp).  Returns (ms per step, wall seconds, the event lists of the stamped
    steps)."""
    stamped = [i % every == 0 for i in range(steps)]
    evs = [[torch.cuda.Event(enable_timing=True) if (j in stamp and stamped[i]) else None for j in range(n_events)]
           for i in range(steps)]
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for e in [t0, t1] + [e for es in evs for e in es if e is not None]:
        e.record(stream)     # torch creates the HIP event on its first record: do it before timing
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record(stream)
    for i in range(steps):
        step(i, evs[i])
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps, time.perf_counter() - wall0, [es for i, es in enumerate(evs) if stamped[i]]


def mean_interval(evs, a, b):
    return sum(e[a].elapsed_time(e[b]) for e in evs) / len(evs)


def kernel_breakdown(torch, step, stream, steps, names):
    """Per-kernel times from a pass before the timed steps in which every launch stamps its
    start (and the last its end): start to start of the next launch, so each includes the
    dispatch gap after it.  The pass picks the dominant kernel; value and roofline come
    from the timed steps."""
    n = len(names) + 1
    _, _, evs = time_steps(torch, step, stream, steps, n, range(n))
    return {name: mean_interval(evs, j, j + 1) for j, name in enumerate(names)}


# In the timed steps the dominant kernel's launch stamps its own start and end on every
# STAMP_EVERY-th step (steps 0, 4, 8, ...: 5 of the default 20), and the roofline takes the
# mean duration of those launches; the other steps run without events.
STAMP_EVERY = 4


def timed_dominant(torch, step, stream, steps, names, dominant):
    """The timed steps: (ms per step, wall seconds, the dominant kernel's mean duration in
    ms, measured on the stamped ones of the same steps from the events its launch stamps)."""
    j = names.index(dominant)
    ms_step, wall, evs = time_steps(torch, step, stream, steps, len(names) + 1, (j, j + 1), STAMP_EVERY)
    return ms_step, wall, mean_interval(evs, j, j + 1)


FORWARD_SOURCES = ("kata_common.h", "kata_chunk.h", "kata_scan.h")
FORWARD_HOST_END = "kata_status validate_flash("


def source_hash(extra=()) -> str:
    """Hash of what the chunked forward's kernels and their launch plan are built from:
    the three device headers they live in and the host code of kata.hip up to the first
    entry point of another path (plus the headers in ``extra``, and then all of kata.hip,
    for another path).  Counters recorded under another hash are not reused."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "kernelized_linear_attention_kata_amd", "csrc")
    for name in FORWARD_SOURCES + tuple(extra):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    with open(os.path.join(csrc, "kata.hip"), "r") as f:
        host = f.read()
    cut = host.find(FORWARD_HOST_END) if not extra else -1
    h.update(b"kata.hip")
    h.update((host[:cut] if cut > 0 else host).encode())
    return h.hexdigest()[:16]


# Headers each bench mode's kernels live in; the mode's counters are keyed by their hash
# together with all of kata.hip (the forward keeps its narrower hash, see source_hash).
PATH_HEADERS = {"decay": ("kata_chunk.h",), "backward": ("kata_bwd.h",), "flash": ("kata_flash.h",),
                "delta": ("kata_delta.h",), "delta_seq": ("kata_delta.h",), "decode": ("kata_decode.h",), "decode_delta": ("kata_delta.h",),
                "decode_delta_packed": ("kata_delta.h", "kata_decode.h")}


def path_hash(mode: str) -> str:
    if mode in ("forward", "forward_precise", "forward_seq", "mid", "lm340m"):
        return source_hash()
    if mode.startswith(("m", "sigma")):
        return source_hash(("kata_chunk.h",))
    if mode.startswith("decode_"):
        return source_hash(PATH_HEADERS.get(mode, ("kata_decode.h",)))
    return source_hash(PATH_HEADERS[mode])


def mode_traffic(mode: str, kernel: str):
    """Recorded HBM bytes per launch of ``kernel`` for a bench mode (None if not current)."""
    fname = "hbm_counters.json" if mode == "forward" else f"hbm_counters_{mode}.json"
    return recorded_traffic(fname, path_hash(mode), kernel)


def recorded_traffic(fname: str, src: str, kernel: str):
    """HBM bytes per launch of ``kernel`` from a committed FETCH_SIZE/WRITE_SIZE summary,
    or None when the summary is missing or was recorded for other kernel sources."""
    path = os.path.join(ROOT, "profiles", fname)
    try:
        cnt = json.load(open(path))
        if cnt.get("source_hash") != src:
            return None
        return cnt["kernels"][kernel]["hbm_bytes_per_launch"]
    except (OSError, ValueError, KeyError):
        return None


def algorithmic_bytes(B, H, T, d, dv, n_leaf, in_bytes, out_bytes, decay=False, factors=1, scan=True):
    """Bytes each kernel must move at minimum (per launch), by the byte model of the path
    (decay: the log-gates, 4 B per token-head, read by the state and intra kernels, and
    one float per leaf; factors: g leaf states per leaf, the tokens still read once).
    scan=False: the plan runs no scan (kata_forward_plan's scanned = 0); the intra pass's
    workgroup of leaf g reads the states of leaves 0 .. g-1 and the last one writes the
    final state."""
    E = 144 * dv + 256                    # packed leaf state block (S slots + Z), floats
    states = factors * B * H * n_leaf * E * 4
    scanned = factors * B * H * n_leaf * (E - 8 * dv) * 4   # the forward scan skips the 8 * dv unused slots
    final = factors * B * H * 256 * (dv + 1) * 4
    tok = B * H * T
    g = tok * 4 if decay else 0
    gl = B * H * n_leaf * 4 if decay else 0
    if not scan:
        return {
            "kata_chunk_state": tok * (d + dv) * in_bytes + states,
            "kata_state_scan": 0,
            "kata_chunk_intra": (tok * (2 * d + dv) * in_bytes + tok * dv * out_bytes
                                 + B * H * (n_leaf * (n_leaf - 1) // 2) * E * 4 + final),
        }
    return {
        "kata_chunk_state": tok * (d + dv) * in_bytes + states + g + gl,
        "kata_state_scan": 2 * scanned + final + gl,
        "kata_chunk_intra": tok * (2 * d + dv) * in_bytes + states + tok * dv * out_bytes + g,
    }


def algorithmic_flops(B, H, T, d, dv, C, factors=1, cross=False):
    """Useful flops per launch (136 distinct packed features, causal half of the score tile;
    every PSD factor does the one-factor work; cross: the summed factors' g*g score tiles)."""
    D = 136
    tok = B * H * T * factors
    proj = 2 * d * 16
    tiles = factors if cross else 1
    return {
        "kata_chunk_state": tok * (proj + 2 * D * (dv + 1)),
        "kata_state_scan": 0,
        "kata_chunk_intra": tok * (2 * proj + 2 * D * (dv + 1) + 2 * D * (dv + 1)
                                   + tiles * (C + 1) * (16 + dv + 1)),
    }


def cpu_baseline(case, stride):
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import kata_oracle as O
    from kernelized_linear_attention_kata_amd import inputs as I

    q = O.bf16_bits_to_f64(I.bf16_bits(case.q))
    k = O.bf16_bits_to_f64(I.bf16_bits(case.k))
    v = O.bf16_bits_to_f64(I.bf16_bits(case.v))
    P = case.P.double().cpu().numpy()
    rows = np.arange(stride - 1, case.T, stride)
    t0 = time.perf_counter()
    O.forward_quadratic(q, k, v, P, rows=rows)
    dt = time.perf_counter() - t0
    est_full = dt * case.T / len(rows)
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    return {
        "value": case.B * case.T / est_full,
        "unit": "tokens/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"fp64 O(T^2) oracle on every {stride}th query row ({len(rows)} rows) of all "
                   f"{case.H} heads, {dt:.1f} s measured; whole-workload time extrapolated x{case.T / len(rows):.0f} "
                   f"(stride sampling keeps the mean causal prefix at T/2)"),
        "seconds": dt,
        "host_cpus": os.cpu_count(),
    }


def decay_cpu_baseline(case, lam, T_sample=16384, heads=8):
    """The oracle's O(T^2) decay-gated forward on the first T_sample tokens of `heads` heads,
    extrapolated to the whole workload by its T^2 cost."""
    from threadpoolctl import threadpool_info

    from oracle import kata_oracle as O
    from kernelized_linear_attention_kata_amd import inputs as I

    hs = slice(0, heads)
    q = O.bf16_bits_to_f64(I.bf16_bits(case.q[:, hs, :T_sample]))
    k = O.bf16_bits_to_f64(I.bf16_bits(case.k[:, hs, :T_sample]))
    v = O.bf16_bits_to_f64(I.bf16_bits(case.v[:, hs, :T_sample]))
    P = case.P[hs].double().cpu().numpy()
    lm = lam[:, hs, :T_sample].double().cpu().numpy()
    t0 = time.perf_counter()
    O.forward_decay_quadratic(q, k, v, P, lm)
    dt = time.perf_counter() - t0
    scale = (case.T / T_sample) ** 2 * (case.H / heads)
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    return {"value": case.B * case.T / (dt * scale), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": (f"fp64 O(T^2) decay-gated oracle on the first {T_sample} tokens of {heads} of {case.H} heads, "
                       f"{dt:.1f} s measured; whole-workload time extrapolated x{scale:.0f} by the T^2 cost")}


def mg_cpu_baseline(case, P, T_sample=16384, heads=8, summed=False):
    """The oracle's O(T^2) KATA-Mg (or, summed, KATA-Sigma-g) forward on the first T_sample
    tokens of `heads` heads, extrapolated to the whole workload by its T^2 cost."""
    from threadpoolctl import threadpool_info

    from oracle import kata_oracle as O
    from kernelized_linear_attention_kata_amd import inputs as I

    hs = slice(0, heads)
    q = O.bf16_bits_to_f64(I.bf16_bits(case.q[:, hs, :T_sample]))
    k = O.bf16_bits_to_f64(I.bf16_bits(case.k[:, hs, :T_sample]))
    v = O.bf16_bits_to_f64(I.bf16_bits(case.v[:, hs, :T_sample]))
    t0 = time.perf_counter()
    (O.forward_sg_quadratic if summed else O.forward_mg_quadratic)(q, k, v, P[hs].double().cpu().numpy())
    dt = time.perf_counter() - t0
    scale = (case.T / T_sample) ** 2 * (case.H / heads)
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    return {"value": case.B * case.T / (dt * scale), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": (f"fp64 O(T^2) KATA-{'Sigma-g' if summed else 'Mg'} oracle (g={P.shape[1]}) on the first "
                       f"{T_sample} tokens of {heads} of "
                       f"{case.H} heads, {dt:.1f} s measured; whole-workload time extrapolated x{scale:.0f} by the "
                       f"T^2 cost")}


DELTA_DECODE_METRIC = ("DeltaKATA decode tokens/sec: 256 streams x 16 heads, fp32 state (p=16, dv=64), "
                       "1024 steps after an 8192-token prefill (1 GPU)")
DECODE_METRIC = ("KATA decode tokens/sec: 256 streams x 16 heads, fp32 state (p=16, dv=64), "
                 "1024 steps after an 8192-token prefill (1 GPU)")


def decode_cpu_baseline(dc, budget_s=10.0, delta=False, betas=None, factors=None):
    """The oracle's decode step (or DeltaKATA decode step) on the host over the same
    streams, steps until budget_s."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import kata_oracle as O
    from kernelized_linear_attention_kata_amd import inputs as I

    N, H, dv = dc.N, dc.H, dc.dv
    rows = 256 * (factors[0].shape[1] if factors is not None and factors[1] == "concat" else 1)
    S = np.zeros((N, H, rows, dv))
    z = np.zeros((N, H, rows))
    P = (factors[0] if factors is not None else dc.P).double().cpu().numpy()
    steps = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s and steps < dc.steps:
        q = O.bf16_bits_to_f64(I.bf16_bits(dc.q[steps]))
        k = O.bf16_bits_to_f64(I.bf16_bits(dc.k[steps]))
        v = O.bf16_bits_to_f64(I.bf16_bits(dc.v[steps]))
        if delta:
            _, S = O.delta_decode_reference(S, q, k, v, P, betas[steps].double().cpu().numpy())
        elif factors is not None:
            _, S, z = O.decode_factors_reference(S, z, q, k, v, P, factors[1])
        else:
            _, S, z = O.decode_reference(S, z, q, k, v, P)
        steps += 1
    dt = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    return {"value": N * steps / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"fp64 oracle {'DeltaKATA ' if delta else ('factor ' if factors is not None else '')}decode step "
                      f"over all {N} streams x {H} heads, "
                      f"first {steps} steps "
                      f"({dt:.1f} s); the cost per step does not depend on the state's values"}


FLASH_METRIC = ("KATA flash-style O(T^2) causal forward tokens/sec, 340M-layer shape "
                "B=8 H=16 T=2048 d=dv=64 p=16, bf16 (1 GPU)")


def flash_algorithmic_flops(B, H, T, d=64, dv=64, p=16):
    """Useful flops: per causal pair 2p (score) + 2dv (weighted values) + 2 (denominator);
    per token and head the two projections 2 * 2pd."""
    pairs = B * H * T * (T + 1) // 2
    return pairs * (2 * p + 2 * dv + 2) + B * H * T * 4 * p * d


def bench_flash(args):
    import torch
    import kernelized_linear_attention_kata_amd as kata
    from kernelized_linear_attention_kata_amd import inputs as I

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    nb = max(1, args.batches)
    seed0 = I.WORKLOADS["lm340m"]["seed"]
    cases = [I.make_forward("lm340m", device=dev, seed=seed0 + b) for b in range(nb)]
    c0 = cases[0]
    B, H, T, d, dv = c0.B, c0.H, c0.T, c0.d, c0.dv
    ws = torch.empty(kata.flash_workspace_bytes(B, H, T), dtype=torch.uint8, device=dev)
    ys = [torch.empty((B, H, T, dv), dtype=torch.bfloat16, device=dev) for _ in range(nb)]
    stream = torch.cuda.current_stream(dev)

    def step(i, events=None):
        c = cases[i % nb]
        kata.flash_forward(c.q, c.k, c.v, c.P, y=ys[i % nb], workspace=ws, stream=stream, events=events)

    settle0 = time.perf_counter()
    n_settle = 0
    while time.perf_counter() - settle0 < args.settle_s:
        for _ in range(8):
            step(n_settle)
            n_settle += 1
        torch.cuda.synchronize()
    for i in range(args.warmup):
        step(i)
    names = ("kata_flash_prep", "kata_flash_attn")
    split = kernel_breakdown(torch, step, stream, args.steps, names)
    ms_step, _, attn_ms = timed_dominant(torch, step, stream, args.steps, names, "kata_flash_attn")
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    flops = flash_algorithmic_flops(B, H, T)
    attn_flops = flops - B * H * T * 4 * 16 * d
    achieved = attn_flops / (attn_ms / 1e3) / 1e12

    # the chunked path on the same inputs, for comparison (same settle state)
    wsc = torch.empty(kata.forward_workspace_bytes(B, H, T, d, dv, 64), dtype=torch.uint8, device=dev)
    for i in range(5):
        c = cases[i % nb]
        kata.forward(c.q, c.k, c.v, c.P, chunk=64, y=ys[i % nb], workspace=wsc, stream=stream)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(args.steps):
        c = cases[i % nb]
        kata.forward(c.q, c.k, c.v, c.P, chunk=64, y=ys[i % nb], workspace=wsc, stream=stream)
    t1.record(stream)
    torch.cuda.synchronize()
    chunked_ms = t0.elapsed_time(t1) / args.steps

    result = {
        "metric": FLASH_METRIC, "value": B * T / (ms_step / 1e3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": f"synthetic ({nb} distinct seeded batches, cycled per step)",
        "config": {"workload": f"flash-style O(T^2) forward (no state), 340M-layer inputs: B={B} H={H} T={T} "
                               f"d=dv={d} p=16, per-head P, unit-norm keys, bf16",
                   "global_batch": B, "seq_len": T, "heads": H},
        "roofline": {"bound": "mfma", "kernel": "kata_flash_attn", "achieved": round(achieved, 1),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": mode_traffic("flash", "kata_flash_attn"), "flops_per_launch": attn_flops},
        "kernels": {"kata_flash_prep": {"ms": round(split["kata_flash_prep"], 4)},
                    "kata_flash_attn": {"ms": round(split["kata_flash_attn"], 4), "ms_timed_steps": round(attn_ms, 4)}},
        "mode": "flash", "source_hash": path_hash("flash"),
        "chunked_path_ms_per_step": round(chunked_ms, 4),
        "settle": {"seconds": round(time.perf_counter() - settle0, 3), "steps": n_settle},
    }
    if not args.no_cpu_baseline:
        cb = cpu_baseline(c0, 1)   # the whole 340M-layer workload: every query row
        result["cpu_baseline"] = {kk: cb[kk] for kk in ("value", "unit", "cores", "kind", "sample")}
    print(json.dumps(result), flush=True)


def bench_decode(args):
    import torch
    import kernelized_linear_attention_kata_amd as kata
    from kernelized_linear_attention_kata_amd import inputs as I

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    delta = bool(args.delta)
    G = args.factors
    fmode = args.factor_mode
    packed = bool(args.packed)
    if delta and G > 1:
        print("bench.py --decode takes --delta or --factors, not both", file=sys.stderr)
        sys.exit(2)
    dc = I.make_decode(device=dev, N=args.streams, T_prefill=args.prefill)
    N, H, d, dv, T0, steps = dc.N, dc.H, dc.d, dc.dv, dc.T_prefill, dc.steps
    prefill = None
    if delta:
        beta0 = I.make_beta(N, H, T0, seed=4, device=dev)
        betas = I.make_beta(steps, N, H, seed=5, device=dev)
        pf0, pf1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        kata.forward_delta(dc.q0, dc.k0, dc.v0, dc.P, beta0, return_state=True)      # untimed first call
        pf0.record()
        _, S0 = kata.forward_delta(dc.q0, dc.k0, dc.v0, dc.P, beta0, return_state=True)
        pf1.record()
        torch.cuda.synchronize()
        pms = pf0.elapsed_time(pf1)
        if packed:        # the delta-rule export has equal mirror rows: packing it is exact
            S0 = kata.state_pack(S0)
        pbytes = N * H * (T0 * (2 * d + dv) * 2 + T0 * (dv * 2 + 4) + 256 * dv * 4)
        prefill = {"kernel": "kata_delta_recurrent", "tokens": N * T0, "ms": round(pms, 3),
                   "tokens_per_s": N * T0 / (pms / 1e3), "hbm_GBps": round(pbytes / (pms / 1e3) / 1e9, 1)}
        z0 = None
    elif G > 1:
        PF = I.make_factor_projections(H, G, d, seed=4, device=dev)
        _, S0, z0 = kata.forward_factors(dc.q0, dc.k0, dc.v0, PF, fmode, return_state=True)
        if packed:        # each factor block packed as a state of its own
            nb = G if fmode == "concat" else 1
            S0, z0 = kata.state_pack(S0.reshape(N, H * nb, 256, dv), z0.reshape(N, H * nb, 256))
            S0, z0 = S0.reshape(N, H, nb * 136, dv), z0.reshape(N, H, nb * 136)
    else:
        _, S0, z0 = kata.forward(dc.q0, dc.k0, dc.v0, dc.P, chunk=64, return_state=True)
        if packed:        # the export has equal mirror rows: packing it is exact
            S0, z0 = kata.state_pack(S0, z0)
    S = torch.empty_like(S0)
    z = torch.empty_like(z0) if z0 is not None else None
    ys = torch.empty((steps, N, H, dv), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    if delta and packed:
        def run(j):
            kata.decode_step_delta_packed(S, dc.q[j], dc.k[j], dc.v[j], dc.P, betas[j], y=ys[j], stream=stream)
    elif delta:
        def run(j):
            kata.decode_step_delta(S, dc.q[j], dc.k[j], dc.v[j], dc.P, betas[j], y=ys[j], stream=stream)
    elif G > 1 and packed:
        def run(j):
            kata.decode_step_factors_packed(S, z, dc.q[j], dc.k[j], dc.v[j], PF, fmode, y=ys[j], stream=stream)
    elif G > 1:
        def run(j):
            kata.decode_step_factors(S, z, dc.q[j], dc.k[j], dc.v[j], PF, fmode, y=ys[j], stream=stream)
    elif packed:
        def run(j):
            kata.decode_step_packed(S, z, dc.q[j], dc.k[j], dc.v[j], dc.P, y=ys[j], stream=stream)
    else:
        def run(j):
            kata.decode_step(S, z, dc.q[j], dc.k[j], dc.v[j], dc.P, y=ys[j], stream=stream)

    def reset():
        S.copy_(S0)
        if z is not None:
            z.copy_(z0)

    reset()
    settle0 = time.perf_counter()
    n_settle = 0
    while time.perf_counter() - settle0 < args.settle_s:
        for _ in range(16):
            run(n_settle % steps)
            n_settle += 1
        torch.cuda.synchronize()
    reset()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream); e1.record(stream)
    torch.cuda.synchronize()
    e0.record(stream)
    for j in range(steps):
        run(j)
    e1.record(stream)
    torch.cuda.synchronize()
    total_ms = e0.elapsed_time(e1)
    ms_step = total_ms / steps
    state_bytes = S.numel() * 4 + (z.numel() * 4 if z is not None else 0)
    step_bytes = 2 * state_bytes + N * H * (2 * d + dv) * 2 + N * H * dv * 4 + (N * H * 4 if delta else 0)
    achieved = step_bytes / (ms_step / 1e3) / 1e9
    kernel = ("kata_delta_recurrent (T=1, in place)" if delta
              else ("kata_decode_step_packed" if packed
                    else ("kata_decode_step_factors" if G > 1 else "kata_decode_step")))
    fname = {"concat": f"KATA-M{G} ", "sum": f"KATA-Sigma{G} "}[fmode] if G > 1 else ""
    mode = ("decode_delta" if delta else
            (f"decode_{'m' if fmode == 'concat' else 'sigma'}{G}" if G > 1 else "decode")) + ("_packed" if packed else "")
    src = path_hash(mode)
    # recorded counters are for the decode workload itself (256 streams)
    traffic = mode_traffic(mode, kernel.split(" ")[0]) if N == 256 else None
    rows = 256 * (G if (G > 1 and fmode == "concat") else 1)
    prefill_fn = "kata_forward_delta" if delta else ("kata_forward_factors" if G > 1 else "kata_forward")
    state_desc = (f"packed symmetric fp32 state [{N},{H},{rows * 136 // 256},{dv}]{'' if delta else ' + z'} "
                  f"(kata_state_pack of the export)" if packed
                  else f"canonical fp32 state [{N},{H},{rows},{dv}]{'' if delta else ' + z'}")
    workload = (f"recurrent {'DeltaKATA ' if delta else fname}decode: {N} streams x {H} heads, d=dv={d}, p=16, "
                f"{state_desc}, prefill T={T0} by "
                f"{prefill_fn}, {steps} steps, every 4th key repeating an earlier one"
                + (", beta uniform in [0.5, 1]" if delta else "")
                + (f", {G} PSD factors per head (P [16,{G},16,64])" if G > 1 else ""))
    result = {
        "metric": (DELTA_DECODE_METRIC if delta else
                   (DECODE_METRIC.replace("KATA decode", f"{fname.strip()} decode", 1) if G > 1 else DECODE_METRIC)
                   ).replace("256 streams", f"{N} streams").replace("8192-token", f"{T0}-token"),
        "value": N * steps / (total_ms / 1e3),
        "unit": "tokens/s", "n_gpus": 1,
        "steps": steps, "warmup": 0, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16 q/k/v, f32 state", "data": "synthetic",
        "config": {"workload": workload, "streams": N, "heads": H},
        "roofline": {"bound": "hbm", "kernel": kernel, "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "bytes_per_step": step_bytes},
        "mode": mode, "source_hash": src,
        "settle": {"seconds": round(time.perf_counter() - settle0, 3), "steps": n_settle},
    }
    if prefill is not None:
        result["prefill"] = prefill
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = decode_cpu_baseline(dc, delta=delta, betas=betas if delta else None,
                                                     factors=(PF, fmode) if G > 1 else None)
    print(json.dumps(result), flush=True)


DELTA_FWD_METRIC = ("DeltaKATA causal fwd tokens/sec at T=131072, chunked (WY) form (1 GPU)")


def delta_cpu_baseline(case, beta, T_sample=65536, heads=8):
    """The oracle's DeltaKATA token recurrence on the first T_sample tokens of `heads` heads,
    extrapolated linearly (the recurrence costs the same per token)."""
    from threadpoolctl import threadpool_info

    from oracle import kata_oracle as O
    from kernelized_linear_attention_kata_amd import inputs as I

    hs = slice(0, heads)
    q = O.bf16_bits_to_f64(I.bf16_bits(case.q[:, hs, :T_sample]))
    k = O.bf16_bits_to_f64(I.bf16_bits(case.k[:, hs, :T_sample]))
    v = O.bf16_bits_to_f64(I.bf16_bits(case.v[:, hs, :T_sample]))
    t0 = time.perf_counter()
    O.delta_recurrence(q, k, v, case.P[hs].double().cpu().numpy(), beta[:, hs, :T_sample].double().cpu().numpy())
    dt = time.perf_counter() - t0
    scale = (case.T / T_sample) * (case.H / heads)
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    return {"value": case.B * case.T / (dt * scale), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": (f"fp64 DeltaKATA token-recurrence oracle on the first {T_sample} tokens of {heads} of "
                       f"{case.H} heads, {dt:.1f} s measured; whole-workload time extrapolated x{scale:.0f} "
                       f"(linear in T)")}


def bench_delta_forward(args):
    """DeltaKATA forward on the long-context workload: the chunked form timed per kernel
    (events from the launches), the token-recurrent form timed once beside it."""
    import torch
    import kernelized_linear_attention_kata_amd as kata
    from kernelized_linear_attention_kata_amd import inputs as I

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    nb = max(1, args.batches)
    seed0 = I.WORKLOADS["long"]["seed"]
    cases = [I.make_forward("long", device=dev, seed=seed0 + b) for b in range(nb)]
    betas = [I.make_beta(c.B, c.H, c.T, seed=seed0 + b, device=dev) for b, c in enumerate(cases)]
    case = cases[0]
    B, H, T, d, dv = case.B, case.H, case.T, case.d, case.dv
    plan = kata.forward_delta_chunked_plan(B, H, T, d, dv, scan=args.scan, scan_leaf=args.leaf)
    wsb = kata.forward_delta_chunked_workspace_bytes(B, H, T, d, dv, scan=args.scan, scan_leaf=args.leaf)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    ys = [torch.empty((B, H, T, dv), dtype=torch.bfloat16, device=dev) for _ in range(nb)]
    stream = torch.cuda.current_stream(dev)

    def step(i, events=None):
        c = cases[i % nb]
        kata.forward_delta_chunked(c.q, c.k, c.v, c.P, betas[i % nb], y=ys[i % nb], workspace=ws, stream=stream,
                                   events=events, scan=args.scan, scan_leaf=args.leaf)

    settle0 = time.perf_counter()
    n_settle = 0
    while time.perf_counter() - settle0 < args.settle_s:
        step(n_settle)
        n_settle += 1
        torch.cuda.synchronize()
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    names = ("kata_delta_prep", "kata_delta_chunk")
    split = kernel_breakdown(torch, step, stream, args.steps, names)
    prep_ms = split["kata_delta_prep"]
    ms_step, _, walk_ms = timed_dominant(torch, step, stream, args.steps, names, "kata_delta_chunk")
    # the token-recurrent form once, for comparison
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    r0.record(stream)
    kata.forward_delta(case.q, case.k, case.v, case.P, betas[0], y=ys[0], stream=stream)
    r1.record(stream)
    torch.cuda.synchronize()
    rec_ms = r0.elapsed_time(r1)
    tok = B * H * T
    n_chunks = (T + 63) // 64
    nseg, seg_chunks = plan["segments"], plan["segment_chunks"]
    dmode = "delta_seq" if args.scan == "sequential" else "delta"
    if nseg > 1:
        walk_how = (f"each head's walk cut into {nseg} segments of {seg_chunks} chunks: the affine maps of all but the last segment "
                    f"({(dv + 144) // 16} column blocks each) side by side, their chain, then the segments' walks "
                    f"side by side, {B * H * nseg * (dv // 16)} workgroups")
    else:
        walk_how = f"{n_chunks} chunks per head walked in order by {dv // 16} workgroups per head"
    prep_bytes = tok * (2 * d * 2 + 4) + tok * 2 * 16 * 4 + B * H * n_chunks * 64 * 64 * 4
    walk_bytes = tok * (2 * 16 * 4 + dv * 2 + 4 + dv * 2) + B * H * n_chunks * 64 * 64 * 4
    # useful walk flops per chunk and 16-column block: K^S and Q^S (2 x 64x256x16), T X (64x64x16),
    # the causal score tile (64x64x16 / 2) times E (64x64x16 / 2), K^^T E (256x64x16); x2 per MAC
    walk_flops = B * H * n_chunks * (dv // 16) * 2 * (2 * 64 * 256 * 16 + 64 * 64 * 16 + 64 * 64 * 16 + 256 * 64 * 16)
    walk_tflops = walk_flops / (walk_ms / 1e3) / 1e12
    result = {
        "metric": DELTA_FWD_METRIC, "value": B * T / (ms_step / 1e3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16 q/k/v/y, f32 state (hi/lo bf16 MFMA products)",
        "data": f"synthetic ({nb} distinct seeded batches, cycled per step)",
        "config": {"workload": (f"long-context DeltaKATA forward: B={B} H={H} T={T} d=dv={d} p=16, beta uniform in "
                                f"[0.5, 1], chunk 64 ({walk_how})"),
                   "global_batch": B, "seq_len": T, "heads": H, "chunk": 64, "batches_cycled": nb},
        "roofline": {"bound": "mfma", "kernel": "kata_delta_chunk", "achieved": round(walk_tflops, 2),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(walk_tflops / MFMA_BF16_PEAK_TFLOPS, 5),
                     "traffic": (mode_traffic(dmode, "kata_delta_chunk") if args.leaf == 0 else None),
                     "note": ("useful flops of the walk (the one-walk form's work; segment maps not counted); "
                              "the walk is a dependency chain over the chunks of a segment: bound by per-chunk "
                              "latency, not by either peak")},
        "kernels": {"kata_delta_prep": {"ms": round(prep_ms, 4), "alg_bytes": prep_bytes,
                                        "alg_GBps": round(prep_bytes / (prep_ms / 1e3) / 1e9, 1)},
                    "kata_delta_chunk": {"ms": round(split["kata_delta_chunk"], 4), "ms_timed_steps": round(walk_ms, 4),
                                         "alg_bytes": walk_bytes,
                                         "alg_GBps": round(walk_bytes / (walk_ms / 1e3) / 1e9, 1),
                                         "alg_TFLOPs": round(walk_tflops, 2),
                                         "us_per_chunk": round(walk_ms * 1e3 / n_chunks, 3)}},
        "mode": dmode, "source_hash": path_hash(dmode),
        "plan": plan,
        "recurrent_form": {"kernel": "kata_delta_recurrent", "ms": round(rec_ms, 3),
                           "tokens_per_s": B * T / (rec_ms / 1e3)},
        "settle": {"seconds": round(time.perf_counter() - settle0, 3), "steps": n_settle},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = delta_cpu_baseline(case, betas[0])
    print(json.dumps(result), flush=True)



BWD_METRIC = ("KATA causal backward (dq, dk, dv, dP) tokens/sec at T=131072, chunked-state form "
              "+ % of HBM peak (1 GPU)")
BWD_KERNELS = ("kata_chunk_state", "kata_state_scan", "kata_bwd_query", "kata_bwd_rstate", "kata_state_scan(rev)",
               "kata_bwd_key", "kata_bwd_dp_reduce")


WORKLOAD_METRIC = "KATA causal fwd tokens/sec, {what} (1 GPU)"
WORKLOAD_WHAT = {
    "mid": "mid workload B=4 H=8 T=4096 d=dv=64 p=16 bf16, chunk 64, + % of HBM peak",
    "lm340m": ("340M-LM-shaped attention layer B=8 H=16 T=2048 d=dv=64 p=16 bf16 (per-head P, unit keys), "
               "chunk 64, + % of HBM peak"),
}
FLUSH_BYTES = 512 << 20


def bench_workload(args):
    """The chunked forward on the mid or the 340M-layer workload.  Their inputs and leaf
    states (about 80 MB and 130 MB per step) fit in the 256 MB last-level cache, so each is
    timed twice: warm (one batch repeated, everything cache-resident) and flushed (a 512 MB
    read of a scratch tensor before every step, so the step starts from HBM; a read, not a
    write, so the step does not also pay for writing back the flush's dirty lines).
    Each flushed step is timed from the start of its first kernel to the end of its last
    (events the launches stamp), which leaves the flush out.  value and roofline are the
    flushed ones; the warm figures come beside them."""
    import torch
    import kernelized_linear_attention_kata_amd as kata
    from kernelized_linear_attention_kata_amd import inputs as I

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    nb = max(1, args.batches)
    seed0 = I.WORKLOADS[args.workload]["seed"]
    cases = [I.make_forward(args.workload, device=dev, seed=seed0 + b) for b in range(nb)]
    case = cases[0]
    B, H, T, d, dv, C = case.B, case.H, case.T, case.d, case.dv, 64
    ws_bytes = kata.forward_workspace_bytes(B, H, T, d, dv, C, scan_leaf=args.leaf)
    plan = kata.forward_plan(B, H, T, d, dv, C, scan_leaf=args.leaf)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    ys = [torch.empty((B, H, T, dv), dtype=torch.bfloat16, device=dev) for _ in range(nb)]
    ST = torch.empty((B, H, 256, dv), dtype=torch.float32, device=dev)
    zT = torch.empty((B, H, 256), dtype=torch.float32, device=dev)
    n_leaf = plan["n_leaf"]
    flush = torch.zeros(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    flush_sink = torch.zeros((), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(i, events=None, c=None):
        c = cases[i % nb] if c is None else c
        kata.forward(c.q, c.k, c.v, c.P, chunk=C, y=ys[i % nb], workspace=ws, ST=ST, zT=zT, return_state=True,
                     scan_leaf=args.leaf, stream=stream, events=events)

    settle0 = time.perf_counter()
    n_settle = 0
    while time.perf_counter() - settle0 < args.settle_s:
        for _ in range(8):
            step(n_settle)
            n_settle += 1
        torch.cuda.synchronize()
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # warm: one batch repeated
    warm_step = lambda i, events=None: step(0, events)
    warm_kernels = kernel_breakdown(torch, warm_step, stream, args.steps, KERNELS)
    warm_ms, wall_warm, _ = time_steps(torch, warm_step, stream, args.steps, len(KERNELS) + 1, ())

    # flushed: every step after a 512 MB read (outside the events).  Three
    # passes, each stamping only what it measures (a stamped launch costs a few us of
    # dispatch gap): all launches for the per-kernel breakdown; the state pass's start and
    # the intra pass's end for the step time (no stamp between them); the dominant
    # kernel's start and end for its duration.
    n_ev = len(KERNELS) + 1

    def flushed_pass(stamp):
        evs = [[torch.cuda.Event(enable_timing=True) if j in stamp else None for j in range(n_ev)]
               for _ in range(args.steps)]
        for es in evs:
            for e in es:
                if e is not None:
                    e.record(stream)
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        for i in range(args.steps):
            flush_sink.copy_(flush.sum())
            step(i, evs[i])
        torch.cuda.synchronize()
        return evs, time.perf_counter() - w0

    evs, _ = flushed_pass(range(n_ev))
    flushed_kernels = {name: mean_interval(evs, j, j + 1) for j, name in enumerate(KERNELS)}
    dominant = max(flushed_kernels, key=flushed_kernels.get)
    evs, wall = flushed_pass((0, n_ev - 1))
    flushed_ms = mean_interval(evs, 0, n_ev - 1)
    jd = KERNELS.index(dominant)
    evs, _ = flushed_pass((jd, jd + 1))
    dominant_ms = mean_interval(evs, jd, jd + 1)

    abytes = algorithmic_bytes(B, H, T, d, dv, n_leaf, 2, 2, scan=plan["scanned"])
    aflops = algorithmic_flops(B, H, T, d, dv, C)
    kernels = {}
    for name in KERNELS:
        ms, wms = flushed_kernels[name], warm_kernels[name]
        kernels[name] = {"ms": round(ms, 4), "ms_warm": round(wms, 4),
                         "alg_GBps": round(abytes[name] / (ms / 1e3) / 1e9, 1),
                         "hbm_frac": round(abytes[name] / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                         "alg_TFLOPs": round(aflops[name] / (ms / 1e3) / 1e12, 2),
                         "mfma_frac": round(aflops[name] / (ms / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                         "alg_bytes": abytes[name], "alg_flops": aflops[name]}
    kernels[dominant]["ms_timed_steps"] = round(dominant_ms, 4)
    achieved = abytes[dominant] / (dominant_ms / 1e3) / 1e9
    mode = args.workload
    result = {
        "metric": WORKLOAD_METRIC.format(what=WORKLOAD_WHAT[args.workload]),
        "value": B * T / (flushed_ms / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": flushed_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": (f"synthetic ({nb} distinct seeded batches cycled in the flushed steps; one batch in the warm "
                 "steps)"),
        "config": {"workload": (f"{args.workload} KATA forward: B={B} H={H} T={T} d=dv={d} p=16, bf16 q/k/v, "
                                f"fp32 P/state, chunk {C}, {n_leaf} leaves per sequence "
                                f"({'assoc scan' if plan['scanned'] else 'prefixes summed in the intra pass, no scan'}); "
                                "each step after a 512 MB read that flushes the caches (warm: no flush, one batch)"),
                   "global_batch": B, "seq_len": T, "heads": H, "chunk": C, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": dominant, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": mode_traffic(mode, dominant) if args.leaf == 0 else None},
        "warm": {"value": B * T / (warm_ms / 1e3), "ms_per_step": warm_ms,
                 "dominant_GBps": round(abytes[dominant] / (warm_kernels[dominant] / 1e3) / 1e9, 1)},
        "kernels": kernels,
        "mode": mode, "source_hash": path_hash(mode),
        "wall_s_timed": round(wall + wall_warm, 4),
    }
    if not args.no_cpu_baseline:
        cb = full_cpu_baseline(case)
        result["cpu_baseline"] = {kk: cb[kk] for kk in ("value", "unit", "cores", "kind", "sample")}
    print(json.dumps(result), flush=True)


def full_cpu_baseline(case):
    """The fp64 O(T^2) oracle over the whole workload (every row of every head)."""
    from threadpoolctl import threadpool_info

    from oracle import kata_oracle as O
    from kernelized_linear_attention_kata_amd import inputs as I

    q, k, v = (O.bf16_bits_to_f64(I.bf16_bits(t)) for t in (case.q, case.k, case.v))
    P = case.P.double().cpu().numpy()
    t0 = time.perf_counter()
    O.forward_quadratic(q, k, v, P)
    dt = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    return {"value": case.B * case.T / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"fp64 O(T^2) oracle over the whole workload ({case.B} x {case.H} sequences of {case.T} "
                      f"tokens), {dt:.1f} s"}


def bwd_algorithmic_bytes(B, H, T, d, dv, n_leaf, gy_bytes):
    """Bytes each backward kernel must move per launch under the byte model of the path:
    its token streams (bf16 q, k, v, dq, dk, dv; gy; the (1/den, h) f32 pair per token
    between the walks) plus the leaf states and dP partials it reads or writes."""
    E = 144 * dv + 256
    states = B * H * n_leaf * E * 4
    parts = B * H * n_leaf * 16 * d * 4
    tok = B * H * T
    gy_b = tok * dv * gy_bytes
    return {
        "kata_chunk_state": tok * (d + dv) * 2 + states,
        "kata_state_scan": 2 * states,
        "kata_bwd_query": tok * (2 * d + dv) * 2 + gy_b + tok * d * 2 + tok * 8 + states + parts,
        "kata_bwd_rstate": tok * d * 2 + gy_b + tok * 8 + states,
        "kata_state_scan(rev)": 2 * states,
        "kata_bwd_key": tok * (2 * d + dv) * 2 + gy_b + tok * 8 + tok * (d + dv) * 2 + states + parts,
        "kata_bwd_dp_reduce": 2 * parts + H * 16 * d * 4,
    }


def bwd_cpu_baseline(case, gy, T_sample, heads_sample):
    """The oracle's O(T^2) backward on the first T_sample tokens of heads_sample heads,
    extrapolated to the whole workload by its T^2 cost."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import kata_oracle as O
    from kernelized_linear_attention_kata_amd import inputs as I

    hs = slice(0, heads_sample)
    q = O.bf16_bits_to_f64(I.bf16_bits(case.q[:, hs, :T_sample]))
    k = O.bf16_bits_to_f64(I.bf16_bits(case.k[:, hs, :T_sample]))
    v = O.bf16_bits_to_f64(I.bf16_bits(case.v[:, hs, :T_sample]))
    g = O.bf16_bits_to_f64(I.bf16_bits(gy[:, hs, :T_sample]))
    P = case.P[hs].double().cpu().numpy()
    t0 = time.perf_counter()
    O.backward_quadratic(q, k, v, P, g)
    dt = time.perf_counter() - t0
    scale = (case.T / T_sample) ** 2 * (case.H / heads_sample)
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    return {"value": case.B * case.T / (dt * scale), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": (f"fp64 O(T^2) oracle backward on the first {T_sample} tokens of {heads_sample} of "
                       f"{case.H} heads, {dt:.1f} s measured; whole-workload time extrapolated x{scale:.0f} "
                       f"by the T^2 cost")}


def bench_backward(args):
    import torch
    import kernelized_linear_attention_kata_amd as kata
    from kernelized_linear_attention_kata_amd import inputs as I

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    nb = max(1, args.batches)
    seed0 = I.WORKLOADS["long"]["seed"]
    cases = [I.make_forward("long", device=dev, seed=seed0 + b) for b in range(nb)]
    c0 = cases[0]
    B, H, T, d, dv = c0.B, c0.H, c0.T, c0.d, c0.dv
    gys = [I.make_output_grad(B, H, T, dv, seed=seed0 + b, device=dev) for b in range(nb)]
    ws_bytes = kata.backward_workspace_bytes(B, H, T, d, dv, 64, scan=args.scan, scan_leaf=args.leaf)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    outs = [(torch.empty_like(c0.q), torch.empty_like(c0.k), torch.empty_like(c0.v),
             torch.empty((H, 16, d), dtype=torch.float32, device=dev)) for _ in range(nb)]
    stream = torch.cuda.current_stream(dev)
    E = 144 * dv + 256
    tok = B * H * T
    # workspace = 2 states + (1/den, h) pairs + 2 dP partial sets (each block 256-byte aligned)
    n_leaf = (ws_bytes - tok * 8) // (2 * B * H * (E + 16 * d) * 4)

    def step(i, events=None):
        c = cases[i % nb]
        kata.backward(c.q, c.k, c.v, c.P, gys[i % nb], scan=args.scan, scan_leaf=args.leaf, workspace=ws,
                      out=outs[i % nb], stream=stream, events=events)

    settle0 = time.perf_counter()
    n_settle = 0
    while time.perf_counter() - settle0 < args.settle_s:
        for _ in range(4):
            step(n_settle)
            n_settle += 1
        torch.cuda.synchronize()
    settle_s = time.perf_counter() - settle0
    for i in range(args.warmup):
        step(i)
    per_kernel = kernel_breakdown(torch, step, stream, args.steps, BWD_KERNELS)
    dominant = max(per_kernel, key=per_kernel.get)
    ms_step, _, dom_ms = timed_dominant(torch, step, stream, args.steps, BWD_KERNELS, dominant)
    abytes = bwd_algorithmic_bytes(B, H, T, d, dv, n_leaf, 2)
    kernels = {name: {"ms": round(ms, 4), "alg_bytes": abytes[name],
                      "alg_GBps": round(abytes[name] / (ms / 1e3) / 1e9, 1),
                      "hbm_frac": round(abytes[name] / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4)}
               for name, ms in per_kernel.items()}
    kernels[dominant]["ms_timed_steps"] = round(dom_ms, 4)
    achieved = abytes[dominant] / (dom_ms / 1e3) / 1e9
    step_bytes = sum(abytes.values())
    result = {
        "metric": BWD_METRIC, "value": B * T / (ms_step / 1e3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": f"synthetic ({nb} distinct seeded batches of q, k, v and gy, cycled per step)",
        "config": {"workload": f"long-context KATA backward: B={B} H={H} T={T} d=dv={d} p=16, bf16 q/k/v/gy "
                               f"(dq, dk, dv bf16; dP f32), chunk 64, {args.scan} scans over {n_leaf} leaf "
                               f"states per head",
                   "global_batch": B, "seq_len": T, "heads": H, "chunk": 64, "batches_cycled": nb},
        "roofline": {"bound": "hbm", "kernel": dominant, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": mode_traffic("backward", dominant)},
        "step_alg_GBps": round(step_bytes / (ms_step / 1e3) / 1e9, 1),
        "kernels": kernels,
        "mode": "backward", "source_hash": path_hash("backward"),
        "settle": {"seconds": round(settle_s, 3), "steps": n_settle},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = bwd_cpu_baseline(c0, gys[0], args.bwd_cpu_tokens, 8)
    print(json.dumps(result), flush=True)


def stream_probe(args):
    """Plain torch kernels over 512 MiB fp32 tensors (2 GiB per pattern, eight times the
    last-level cache): a sum (pure read), a copy (1 read : 1 write) and addcmul (3 reads :
    1 write, the intra pass's mix).  Each runs after the usual clock settle, 20 times, timed
    with events; the JSON line gives each pattern's bytes moved per second."""
    import torch
    dev = torch.device("cuda:0")
    n = (512 << 20) // 4
    a, b, c, d = (torch.full((n,), 1.0 + i, device=dev) for i in range(4))
    acc = torch.empty((), device=dev)
    pats = {"read": (lambda: torch.sum(a, dim=0, out=acc), 4 * n),
            "copy_1r1w": (lambda: d.copy_(a), 8 * n),
            "addcmul_3r1w": (lambda: torch.addcmul(a, b, c, out=d), 16 * n)}
    out = {}
    for name, (fn, nbytes) in pats.items():
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < args.settle_s:
            fn()
            torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(20):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 20
        out[name] = {"bytes": nbytes, "ms": round(ms, 4), "GBps": round(nbytes / (ms / 1e3) / 1e9, 1),
                     "frac_of_8TBps": round(nbytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4)}
    print(json.dumps({"probe": "plain torch streaming kernels, 512 MiB fp32 tensors", "patterns": out}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--batches", type=int, default=4, help="distinct input batches cycled over the steps")
    ap.add_argument("--settle-s", type=float, default=0.5,
                    help="seconds of untimed steps before the warmup (clock ramp of an idle GPU)")
    ap.add_argument("--chunk", type=int, default=64, choices=(32, 64, 128))
    ap.add_argument("--workload", default="long", choices=("long", "mid", "lm340m"),
                    help="the chunked forward on the mid or the 340M-layer workload instead (warm and flushed)")
    ap.add_argument("--leaf", type=int, default=0, help="chunks per scan leaf (0 = library default)")
    ap.add_argument("--scan", default="assoc", choices=("assoc", "sequential"))
    ap.add_argument("--precise", action="store_true",
                    help="the KATA_BF16_HILO compute type (hi/lo feature and state operands)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-stride", type=int, default=16)
    ap.add_argument("--decode", action="store_true", help="time the recurrent decode step instead")
    ap.add_argument("--factors", type=int, default=1, choices=(1, 2, 3),
                    help="KATA-Mg: time kata_forward_factors with this many concatenated PSD factors")
    ap.add_argument("--factor-mode", default="concat", choices=("concat", "sum"),
                    help="with --factors: concatenated (KATA-Mg) or summed (KATA-Sigma-g) factors")
    ap.add_argument("--streams", type=int, default=None,
                    help="with --decode: streams (default 256, the decode workload's); 1024 makes the state "
                         "4.3x the 256 MB last-level cache")
    ap.add_argument("--prefill", type=int, default=None,
                    help="with --decode: prefill tokens per stream (default 8192; the step's cost does not "
                         "depend on it)")
    ap.add_argument("--packed", action="store_true",
                    help="with --decode: the step on the packed symmetric state (kata_decode_step_packed)")
    ap.add_argument("--delta", action="store_true",
                    help="the DeltaKATA forward (chunked form) on the long-context workload; with --decode the "
                         "DeltaKATA decode step (prefill by kata_forward_delta)")
    ap.add_argument("--flash", action="store_true", help="time the flash-style O(T^2) forward instead")
    ap.add_argument("--backward", action="store_true", help="time the chunked-state backward instead")
    ap.add_argument("--decay", action="store_true",
                    help="time the decay-gated forward (kata_forward_decay, gates in [0.9, 1]) instead")
    ap.add_argument("--bwd-cpu-tokens", type=int, default=16384,
                    help="prefix length of the oracle's backward sample (CPU baseline of --backward)")
    ap.add_argument("--stream-probe", action="store_true",
                    help="only time plain torch streaming kernels (pure read, 1:1 copy, 3 reads : 1 write) "
                         "over footprints past the last-level cache: the memory system's practical rates")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB five times (reference for HBM counters)")
    args = ap.parse_args()
    if args.stream_probe:
        stream_probe(args)
        return
    if args.copy_calibration:
        # Plain device copies of MIB MiB: the reference for the HBM counters (1 GiB, five
        # copies) and, at small sizes, the time a copy of a kernel's own bytes takes (after
        # a clock settle, 400 copies cycling over 8 buffer pairs).
        import torch
        n = args.copy_calibration * (1 << 20) // 4
        pairs, launches = (8, 400) if args.copy_calibration <= 64 else (1, 5)
        srcs = [torch.ones(n, dtype=torch.float32, device="cuda:0") for _ in range(pairs)]
        dsts = [torch.empty_like(srcs[0]) for _ in range(pairs)]
        if pairs > 1:
            t0 = time.perf_counter()
            while time.perf_counter() - t0 < args.settle_s:
                for i in range(pairs):
                    dsts[i].copy_(srcs[(i + 3) % pairs])
                torch.cuda.synchronize()
        for i in range(launches):
            dsts[i % pairs].copy_(srcs[(i + 3) % pairs])
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "launches": launches}))
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}); "
              "sequences and heads shard across GPUs without exchange and one long sequence by carrying "
              "the state (the resume form), but no multi-GPU run is made here.", file=sys.stderr)
        sys.exit(2)

    if args.decode:
        bench_decode(args)
        return
    if args.delta:
        bench_delta_forward(args)
        return
    if args.flash:
        bench_flash(args)
        return
    if args.backward:
        bench_backward(args)
        return
    if args.workload != "long":
        bench_workload(args)
        return

    import torch
    import kernelized_linear_attention_kata_amd as kata
    from kernelized_linear_attention_kata_amd import inputs as I

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    nb = max(1, args.batches)
    seed0 = I.WORKLOADS["long"]["seed"]
    cases = [I.make_forward("long", device=dev, chunk=args.chunk, seed=seed0 + b) for b in range(nb)]
    case = cases[0]
    B, H, T, d, dv, C = case.B, case.H, case.T, case.d, case.dv, args.chunk
    ws_bytes = kata.forward_workspace_bytes(B, H, T, d, dv, C, scan=args.scan, scan_leaf=args.leaf,
                                            precise=args.precise)
    G = args.factors
    if args.precise and (args.decay or G > 1):
        print("bench.py --precise applies to the plain forward", file=sys.stderr)
        sys.exit(2)
    if (args.decay or G > 1) and C != 64:
        print("bench.py --decay / --factors support chunk 64 only", file=sys.stderr)
        sys.exit(2)
    if G > 1:
        Ps = [I.make_factor_projections(H, G, d, seed=seed0 + b, device=dev) for b in range(nb)]
        wsf = kata.forward_factors_workspace_bytes(B, H, T, G, args.factor_mode)
        ws_bytes = wsf // G if args.factor_mode == "concat" else wsf
        ws = torch.empty(wsf, dtype=torch.uint8, device=dev)
    elif args.decay:
        lams = [I.make_log_decay(B, H, T, seed=seed0 + b, device=dev) for b in range(nb)]
        wsd = kata.forward_decay_workspace_bytes(B, H, T, d, dv, C, scan=args.scan, scan_leaf=args.leaf)
        ws = torch.empty(wsd, dtype=torch.uint8, device=dev)
    else:
        ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    ys = [torch.empty((B, H, T, dv), dtype=torch.bfloat16, device=dev) for _ in range(nb)]
    ST = torch.empty((B, H, 256, dv), dtype=torch.float32, device=dev)
    zT = torch.empty((B, H, 256), dtype=torch.float32, device=dev)
    E = 144 * dv + 256
    n_leaf = ws_bytes // (B * H * E * 4)
    stream = torch.cuda.current_stream(dev)

    def step(i, events=None):
        c = cases[i % nb]
        if G > 1:
            kata.forward_factors(c.q, c.k, c.v, Ps[i % nb], args.factor_mode, chunk=C, y=ys[i % nb], workspace=ws,
                                 stream=stream, events=events)
            return
        if args.decay:
            kata.forward_decay(c.q, c.k, c.v, c.P, lams[i % nb], chunk=C, y=ys[i % nb], workspace=ws,
                               return_state=False, scan=args.scan, scan_leaf=args.leaf, stream=stream, events=events)
            return
        kata.forward(c.q, c.k, c.v, c.P, chunk=C, y=ys[i % nb], workspace=ws, ST=ST, zT=zT, return_state=True,
                     scan=args.scan, scan_leaf=args.leaf, stream=stream, events=events, precise=args.precise)

    settle0 = time.perf_counter()
    n_settle = 0
    while time.perf_counter() - settle0 < args.settle_s:
        for _ in range(8):
            step(n_settle)
            n_settle += 1
        torch.cuda.synchronize()
    settle_s = time.perf_counter() - settle0
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    per_kernel = kernel_breakdown(torch, step, stream, args.steps, KERNELS)
    dominant = max(per_kernel, key=per_kernel.get)
    ms_per_step, wall, dom_ms = timed_dominant(torch, step, stream, args.steps, KERNELS, dominant)
    total_ms = ms_per_step * args.steps

    tokens_per_s = B * T / (ms_per_step / 1e3)
    sg = G > 1 and args.factor_mode == "sum"
    fac_word = "summed" if sg else "concatenated"
    fac_note = f" with {G} {fac_word} PSD factors (P [16,{G},16,64], no state export)" if G > 1 else ""
    scanned = True
    if G == 1 and not args.decay:
        scanned = kata.forward_plan(B, H, T, d, dv, C, scan=args.scan, scan_leaf=args.leaf,
                                    precise=args.precise)["scanned"]
    abytes = algorithmic_bytes(B, H, T, d, dv, n_leaf, 2, 2, decay=args.decay, factors=1 if sg else G, scan=scanned)
    aflops = algorithmic_flops(B, H, T, d, dv, C, factors=G, cross=sg)
    kernels = {}
    for name in KERNELS:
        ms = per_kernel[name]
        kernels[name] = {
            "ms": round(ms, 4),
            "alg_GBps": round(abytes[name] / (ms / 1e3) / 1e9, 1),
            "hbm_frac": round(abytes[name] / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
            "alg_TFLOPs": round(aflops[name] / (ms / 1e3) / 1e12, 2),
            "mfma_frac": round(aflops[name] / (ms / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "alg_bytes": abytes[name],
            "alg_flops": aflops[name],
        }
    kernels[dominant]["ms_timed_steps"] = round(dom_ms, 4)
    achieved = abytes[dominant] / (dom_ms / 1e3) / 1e9
    traffic = None
    mode = (f"{'sigma' if sg else 'm'}{G}" if G > 1
            else ("decay" if args.decay else ("forward_precise" if args.precise else
                                              ("forward_seq" if args.scan == "sequential" else "forward"))))
    src = path_hash(mode)
    # counters are recorded on the default plan (chunk 64, the library's leaf size)
    if C == 64 and args.leaf == 0:
        traffic = mode_traffic(mode, dominant)

    result = {
        "metric": ((SG_METRIC if sg else MG_METRIC).format(g=G) if G > 1
                   else (DECAY_METRIC if args.decay else METRIC)),
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": f"synthetic ({nb} distinct seeded batches, cycled per step)",
        "config": {"workload": (f"long-context KATA{(f'-Sigma{G}' if sg else f'-M{G}') if G > 1 else ''} forward"
                                f"{' (KATA_BF16_HILO: hi/lo feature and state operands)' if args.precise else ''}"
                                f"{' with decay gates in [0.9, 1] (fp32 log-gates)' if args.decay else ''}"
                                f"{fac_note}: "
                                f"B={B} H={H} T={T} d=dv={d} p=16, bf16 q/k/v, fp32 P/state, chunk {C}, "
                                f"{args.scan} scan over {n_leaf} leaf states per head"),
                   "global_batch": B, "seq_len": T, "heads": H, "chunk": C, "batches_cycled": nb,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": dominant, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic},
        "kernels": kernels,
        "mode": mode, "source_hash": src,
        "wall_s_timed": round(wall, 4),
        "settle": {"seconds": round(settle_s, 3), "steps": n_settle},
    }
    if not args.no_cpu_baseline:
        if G > 1:
            cb = mg_cpu_baseline(case, Ps[0], summed=sg)
        elif args.decay:
            cb = decay_cpu_baseline(case, lams[0])
        else:
            cb = cpu_baseline(case, args.cpu_stride)
        result["cpu_baseline"] = {kk: cb[kk] for kk in ("value", "unit", "cores", "kind", "sample")}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

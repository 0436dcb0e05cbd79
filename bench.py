#!/usr/bin/env python3
"""GDN token-mixer benchmark on one MI355X.

One step = one gdn_fwd_chunked call (chunk-local gates, UT transform, W/U,
masked products, state scan, outputs and final states) over the batch
B=4, T=4096, 16 heads, dk=dv=128, bf16 in, fp32 state ("prefill_b4_t4096").
``value`` is that prefill's throughput in Mtok/s with inputs resident in HBM.
The same JSON line also carries
  roofline      the prefill kernel's achieved algorithmic TFLOP/s against the
                2.5 PFLOP/s dense bf16 matrix-core peak, timed with HIP events
                on the launch stream around the K back-to-back launches;
  decode        64 consecutive gdn_decode_step calls on 256 sequences x 32 value
                heads (512 MiB fp32 state): algorithmic GB/s against 8 TB/s;
  verify        gdn_decode_verify, 4 drafted tokens per sequence from the same
                kind of live state: algorithmic GB/s against 8 TB/s;
  epilogue      gdn_output_norm_gate over the prefill output: GB/s against 8 TB/s;
  short_conv    gdn_short_conv with L2 norm over the prefill's q: GB/s against 8 TB/s;
  bwd           gdn_bwd_chunked (all gradients) over the prefill's inputs:
                algorithmic GB/s against 8 TB/s (its 197 flops per algorithmic
                byte sit below the chip's ridge), and its dense-tile TFLOP/s;
  cpu_baseline  the fp64 oracle on the host cores over the same workload.
Inputs are seeded synthetic tensors (linear_attention_token_chunked_amd.inputs).
Every timed loop starts after W untimed steps and at least --warm-seconds of
untimed load, so that it sees the GPU at its steady clocks.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--warm-seconds S] [--no-cpu-baseline] [--all]
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

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 matrix-core peak
PEAK_FP32_TFLOPS = 157.3
PEAK_HBM_GBPS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = {
    "prefill": os.path.join(ROOT, "linear_attention_token_chunked_amd", "csrc", "prefill.hip"),
    "decode": os.path.join(ROOT, "linear_attention_token_chunked_amd", "csrc", "decode.hip"),
    "prefill_save": os.path.join(ROOT, "linear_attention_token_chunked_amd", "csrc", "prefill.hip"),
    "bwd_dstate": os.path.join(ROOT, "linear_attention_token_chunked_amd", "csrc", "bwd.hip"),
    "bwd_dlocal": os.path.join(ROOT, "linear_attention_token_chunked_amd", "csrc", "bwd.hip"),
    "verify": os.path.join(ROOT, "linear_attention_token_chunked_amd", "csrc", "verify.hip"),
    "epilogue": os.path.join(ROOT, "linear_attention_token_chunked_amd", "csrc", "epilogue.hip"),
    "short_conv": os.path.join(ROOT, "linear_attention_token_chunked_amd", "csrc", "conv.hip"),
}
EPILOGUE_WORKLOAD = "epilogue_b4_t4096"
SHORT_CONV_WORKLOAD = "short_conv_q_b4_t4096"


# ------------------------------------------------------------------ algorithmic work
def prefill_flops_per_token(Hqk, Hv, dk, dv, C):
    """Dense-tile flops of the chunked form's products per token: K K^T and Q K^T per
    query/key head; T [K|V], P U, W M, Q M and K^T U per value head."""
    return Hqk * (4 * C * dk) + Hv * (2 * C * (dk + dv) + 2 * C * dv + 6 * dk * dv)


def prefill_bytes(tokens, N, Hqk, Hv, dk, dv, s_in, has_initial, has_final):
    """q, k, v read, o written, g and beta read (fp32), states read/written once."""
    per_tok = 2 * Hqk * dk * s_in + Hv * dv * s_in + Hv * dv * s_in + 8 * Hv
    states = (int(has_initial) + int(has_final)) * N * Hv * dk * dv * 4
    return tokens * per_tok + states


def decode_bytes(N, Hqk, Hv, dk, dv, s_in):
    """Per step: the fp32 state read and written, q, k, v read and o written, g and beta read."""
    return N * Hv * dk * dv * 4 * 2 + N * (2 * Hqk * dk + 2 * Hv * dv) * s_in + N * Hv * 8


def verify_bytes(N, Tv, Hqk, Hv, dk, dv, s_in):
    """Per call: the fp32 state read and written once, and Tv tokens' q, k, v, o, g, beta."""
    return N * Hv * dk * dv * 4 * 2 + Tv * (N * (2 * Hqk * dk + 2 * Hv * dv) * s_in + N * Hv * 8)


def bwd_flops_per_token(Hqk, Hv, dk, dv, C):
    """Dense-tile flops per token of the chunked backward, each product counted once: the forward
    recompute (prefill_flops_per_token), Q K^T and K K^T per query/key head, and per value head
    P^T dO, dO U^T, dZ U^T (2 C^2 dv each), (I + A)^-T dU (C^2 dv), K dM', Q^T dO, K^T dZ, dO M^T,
    dZ M^T, U dM'^T (2 C dk dv each), (dP)K, (dP)^T Q, (D + D^T) K (2 C^2 dk each)."""
    return (prefill_flops_per_token(Hqk, Hv, dk, dv, C) + Hqk * (4 * C * dk)
            + Hv * (7 * C * dv + 6 * C * dk + 12 * dk * dv))


def bwd_bytes(tokens, N, Hqk, Hv, dk, dv, s_in):
    """q, k, v, dO, g, beta read; dq, dk, dv (fp32), dg, dbeta written; the initial state and the final
    state's gradient read and the initial state's gradient written (fp32)."""
    per_tok = 2 * Hqk * dk * s_in + 2 * Hv * dv * s_in + 8 * Hv + 2 * Hqk * dk * 4 + Hv * dv * 4 + 8 * Hv
    return tokens * per_tok + 3 * N * Hv * dk * dv * 4


def source_hash(path):
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch from committed rocprofv3 FETCH_SIZE/WRITE_SIZE runs, or None
    when they are missing or were taken on a different kernel source."""
    try:
        rec = json.load(open(TRAFFIC_FILE))[kernel]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("workload") != workload or rec.get("source_sha256_16") != source_hash(KERNEL_SOURCES[kernel]):
        return None
    return rec.get("bytes_per_launch")


# ------------------------------------------------------------------ CPU baseline
def _oracle_unit(args):
    """Worker: the fp64 oracle on one (sequence, value head) unit."""
    from threadpoolctl import threadpool_limits

    from oracle import recurrent

    q, k, v, g, beta = args
    with threadpool_limits(1):
        recurrent(q, k, v, g, beta)
    return q.shape[1]


def cpu_baseline(inp, workers):
    """Time the oracle over every (sequence, value head) unit of the batch on `workers` processes."""
    import multiprocessing as mp

    import numpy as np

    f = {k: inp[k].float().numpy().astype(np.float64) for k in ("q", "k", "v", "g", "beta")}
    B, T, Hqk, _ = f["q"].shape
    Hv = f["v"].shape[2]
    rep = Hv // Hqk
    units = []
    for b in range(B):
        for h in range(Hv):
            hq = h // rep
            units.append((f["q"][b:b + 1, :, hq:hq + 1], f["k"][b:b + 1, :, hq:hq + 1], f["v"][b:b + 1, :, h:h + 1],
                          f["g"][b:b + 1, :, h:h + 1], f["beta"][b:b + 1, :, h:h + 1]))
    ctx = mp.get_context("fork")  # forked before this process touches the GPU
    t0 = time.perf_counter()
    with ctx.Pool(workers) as pool:
        pool.map(_oracle_unit, units, chunksize=1)
    dt = time.perf_counter() - t0
    tokens = B * T
    return {"value": tokens / dt / 1e6, "unit": "Mtok/s", "cores": workers, "kind": "oracle",
            "sample": f"whole workload: {B}x{T} tokens, all {B * Hv} (sequence, value head) units of the fp64 "
                      f"token recurrence, {dt:.2f} s wall on {workers} processes",
            "seconds": round(dt, 3)}


# ------------------------------------------------------------------ GPU timing
WARM_SECONDS = 1.0  # set from --warm-seconds


def time_launches(fn, steps, warmup, torch):
    """Run fn() warmup times, and on for at least WARM_SECONDS of wall time in all, then time
    exactly `steps` calls back to back: wall clock around the whole loop (synchronised on both
    sides) and one pair of HIP events on the launch stream around it.  Returns the wall time
    (s), the event time per launch (ms) and, from a second loop of `steps` calls with events
    around every launch, the sorted per-launch times (ms).  (Events between launches cost the
    stream a few microseconds each, so the first loop has none.)
    The GPU raises its clocks only after some hundreds of milliseconds of sustained load;
    without the timed warm-up the first launches of a fresh process run up to 15 % slower
    than the steady state."""
    t0 = time.perf_counter()
    n = 0
    while n < warmup or time.perf_counter() - t0 < WARM_SECONDS:
        fn()
        n += 1
        if n % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    mean_ms = e0.elapsed_time(e1) / steps
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in evs:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    per = sorted(a.elapsed_time(b) for a, b in evs)
    return wall, mean_ms, per


def bench_prefill(name, gdn, torch, steps, warmup):
    from linear_attention_token_chunked_amd.inputs import WORKLOADS, make_workload

    w = WORKLOADS[name]
    inp = make_workload(w)
    dev = {k: (v.cuda() if v is not None else None) for k, v in inp.items()}
    B, T, Hqk, dk = dev["q"].shape
    Hv, dv = dev["v"].shape[2], dev["v"].shape[3]
    N = B if dev["cu_seqlens"] is None else dev["cu_seqlens"].shape[0] - 1
    out = torch.empty((B, T, Hv, dv), dtype=dev["q"].dtype, device="cuda")
    fin = torch.empty((N, Hv, dk, dv), dtype=torch.float32, device="cuda")
    ws_bytes = gdn.fwd_chunked_workspace_size(gdn.make_dims(B, T, N, Hqk, Hv, dk, dv, w.chunk, 1.0, dev["q"].dtype))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda") if ws_bytes else None

    def step():
        gdn.fwd_chunked(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], initial_state=dev["initial_state"],
                        cu_seqlens=dev["cu_seqlens"], chunk_size=w.chunk, out=out, final_state=fin, workspace=ws)

    torch.cuda.synchronize()
    c0 = time.perf_counter()
    step()
    torch.cuda.synchronize()
    cold_ms = (time.perf_counter() - c0) * 1e3
    wall, kern_ms, per = time_launches(step, steps, warmup, torch)
    tokens = B * T
    flops = prefill_flops_per_token(Hqk, Hv, dk, dv, w.chunk) * tokens
    nbytes = prefill_bytes(tokens, N, Hqk, Hv, dk, dv, dev["q"].element_size(), dev["initial_state"] is not None,
                           True)
    return {
        "workload": name, "tokens": tokens, "B": B, "T": T, "num_seqs": N, "Hqk": Hqk, "Hv": Hv, "dk": dk, "dv": dv,
        "chunk": w.chunk, "ms_per_step": wall / steps * 1e3, "kernel_ms_mean": kern_ms,
        "kernel_ms_p10": per[len(per) // 10], "kernel_ms_p90": per[(len(per) * 9) // 10], "cold_ms": cold_ms,
        "Mtok_s": tokens / (wall / steps) / 1e6, "flops_per_launch": flops, "bytes_per_launch": nbytes,
        "tflops": flops / (kern_ms * 1e-3) / 1e12, "hbm_gbps": nbytes / (kern_ms * 1e-3) / 1e9,
    }, inp


def bench_decode(gdn, torch, warmup_rounds=1):
    from linear_attention_token_chunked_amd.inputs import WORKLOADS, make_workload

    w = WORKLOADS["decode_n256"]
    inp = make_workload(w)
    dev = {k: v.cuda() for k, v in inp.items()}
    state = dev["state"].clone()
    o = torch.empty((w.N, w.Hv, w.dv), dtype=dev["q"].dtype, device="cuda")
    it = {"t": 0}

    def step():
        t = it["t"] % w.steps
        gdn.decode_step(dev["q"][t], dev["k"][t], dev["v"][t], dev["g"][t], dev["beta"][t], state, out=o)
        it["t"] += 1

    wall, mean_ms, per = time_launches(step, w.steps, warmup_rounds * w.steps, torch)
    us = mean_ms * 1e3
    nbytes = decode_bytes(w.N, w.Hqk, w.Hv, w.dk, w.dv, dev["q"].element_size())
    gbps = nbytes / (us * 1e-6) / 1e9
    traffic = measured_traffic("decode", w.name)
    return {
        "workload": w.name, "N": w.N, "Hqk": w.Hqk, "Hv": w.Hv, "dk": w.dk, "dv": w.dv, "steps": w.steps,
        "us_per_step_mean": us, "us_per_step_median": per[len(per) // 2] * 1e3, "wall_ms_total": wall * 1e3,
        "bytes_per_step": nbytes, "GBps": gbps,
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(gbps / PEAK_HBM_GBPS, 4), "traffic": traffic},
    }


def bench_verify(gdn, torch, steps=20):
    """Multi-token verify (Tv drafted tokens per sequence from a live state), state updated in place."""
    from linear_attention_token_chunked_amd.inputs import WORKLOADS, make_workload

    w = WORKLOADS["verify_n256_t4"]
    inp = make_workload(w)
    dev = {k: v.cuda() for k, v in inp.items()}
    state = dev["state"].clone()
    o = torch.empty((w.N, w.steps, w.Hv, w.dv), dtype=dev["q"].dtype, device="cuda")

    def step():
        gdn.decode_verify(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], state, out=o)

    wall, mean_ms, per = time_launches(step, steps, 2, torch)
    us = mean_ms * 1e3
    nbytes = verify_bytes(w.N, w.steps, w.Hqk, w.Hv, w.dk, w.dv, dev["q"].element_size())
    gbps = nbytes / (us * 1e-6) / 1e9
    return {
        "workload": w.name, "N": w.N, "tokens_per_seq": w.steps, "Hqk": w.Hqk, "Hv": w.Hv, "dk": w.dk, "dv": w.dv,
        "us_per_call_mean": us, "us_per_call_median": per[len(per) // 2] * 1e3,
        "Mtok_s": w.N * w.steps / (us * 1e-6) / 1e6, "bytes_per_call": nbytes, "GBps": gbps,
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(gbps / PEAK_HBM_GBPS, 4), "traffic": measured_traffic("verify", w.name)},
    }


def bench_epilogue(gdn, torch, steps=50):
    """Output epilogue (zero-centred RMSNorm + sigmoid gate) over the prefill_b4_t4096 output."""
    from linear_attention_token_chunked_amd.inputs import make_epilogue

    rows, dv = 4 * 4096 * 16, 128
    dev = {k: v.cuda() for k, v in make_epilogue(rows, dv, "bf16").items()}
    y = torch.empty_like(dev["o"])

    def step():
        gdn.output_norm_gate(dev["o"], dev["z"], dev["w"], out=y)

    wall, mean_ms, per = time_launches(step, steps, 5, torch)
    us = mean_ms * 1e3
    nbytes = 3 * rows * dv * dev["o"].element_size() + dv * 4
    gbps = nbytes / (us * 1e-6) / 1e9
    return {
        "workload": EPILOGUE_WORKLOAD, "what": "prefill_b4_t4096 output (262144 rows x 128, bf16)", "rows": rows,
        "dv": dv, "us_per_call_mean": us, "bytes_per_call": nbytes, "GBps": gbps,
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(gbps / PEAK_HBM_GBPS, 4),
                     "traffic": measured_traffic("epilogue", EPILOGUE_WORKLOAD)},
    }


def bench_short_conv(gdn, torch, steps=50):
    """Pre-mixer short convolution + per-head L2 norm over q (or k) of prefill_b4_t4096."""
    from linear_attention_token_chunked_amd.inputs import make_conv

    B, T, H, hd = 4, 4096, 16, 128
    inp = make_conv(B, T, H, hd, "bf16")
    x, w = inp["x"].cuda(), inp["w"].cuda()
    y = torch.empty_like(x)

    def step():
        gdn.short_conv(x, w, l2norm=True, out=y)

    wall, mean_ms, per = time_launches(step, steps, 5, torch)
    us = mean_ms * 1e3
    nbytes = 2 * x.numel() * x.element_size() + w.numel() * 4
    gbps = nbytes / (us * 1e-6) / 1e9
    return {
        "workload": SHORT_CONV_WORKLOAD,
        "what": "q of prefill_b4_t4096 (4 x 4096 tokens x 16 heads x 128, bf16), width 4, L2 norm",
        "us_per_call_mean": us, "bytes_per_call": nbytes, "GBps": gbps,
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(gbps / PEAK_HBM_GBPS, 4),
                     "traffic": measured_traffic("short_conv", SHORT_CONV_WORKLOAD)},
    }


def bench_bwd(gdn, torch, steps=10):
    """Backward pass (gradients of q, k, v, g, beta and the initial state) over prefill_b4_t4096."""
    from linear_attention_token_chunked_amd.inputs import WORKLOADS, make_cotangents, make_workload

    w = WORKLOADS["prefill_b4_t4096"]
    dev = {k: (v.cuda() if v is not None else None) for k, v in make_workload(w).items()}
    cot = make_cotangents(w.B, w.T, w.Hv, w.dv, w.B, w.dk, w.dtype)
    d_o, d_fin = cot["d_o"].cuda(), cot["d_final"].cuda()
    dims = gdn.make_dims(w.B, w.T, w.B, w.Hqk, w.Hv, w.dk, w.dv, w.chunk, 1.0, dev["q"].dtype)
    ws = torch.empty(gdn.bwd_chunked_workspace_size(dims), dtype=torch.uint8, device="cuda")

    def step():
        gdn.bwd_chunked(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], d_o, initial_state=dev["initial_state"],
                        d_final_state=d_fin, scale=w.dk ** -0.5, workspace=ws)

    wall, mean_ms, per = time_launches(step, steps, 2, torch)
    tokens = w.B * w.T
    flops = bwd_flops_per_token(w.Hqk, w.Hv, w.dk, w.dv, w.chunk) * tokens
    nbytes = bwd_bytes(tokens, w.B, w.Hqk, w.Hv, w.dk, w.dv, dev["q"].element_size())
    tflops = flops / (mean_ms * 1e-3) / 1e12
    gbps = nbytes / (mean_ms * 1e-3) / 1e9
    parts = [measured_traffic(k, w.name) for k in ("prefill_save", "bwd_dstate", "bwd_dlocal")]
    # 198 flops per algorithmic byte, below the chip's 312 (2.5 PFLOP/s over 8 TB/s): the HBM roof is the lower one
    return {
        "workload": w.name, "tokens": tokens, "ms_per_call_mean": mean_ms, "ms_per_call_median": per[len(per) // 2],
        "Mtok_s": tokens / (mean_ms * 1e-3) / 1e6, "flops_per_call": flops, "tflops": tflops,
        "mfma_frac": round(tflops / PEAK_BF16_TFLOPS, 4), "bytes_per_call": nbytes,
        "kernels": "saving prefill, state-gradient scan, local gradients (one call = all three)",
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(gbps / PEAK_HBM_GBPS, 4),
                     "traffic": sum(parts) if all(x is not None for x in parts) else None},
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--warm-seconds", type=float, default=1.0,
                    help="keep warming up (untimed) for at least this long per workload")
    ap.add_argument("--workload", default="prefill_b4_t4096")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--all", action="store_true", help="also time the other prefill workloads (extra field)")
    ap.add_argument("--pmc-calib-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()
    global WARM_SECONDS
    WARM_SECONDS = args.warm_seconds
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the mixer needs no cross-GPU exchange and this build has no "
              "multi-GPU path; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    from linear_attention_token_chunked_amd.inputs import WORKLOADS, make_workload

    cpu = None
    if not args.no_cpu_baseline:
        # before any GPU call: the oracle runs in forked worker processes
        workers = max(1, min(16, len(os.sched_getaffinity(0))))
        cpu = cpu_baseline(make_workload(WORKLOADS[args.workload]), workers)

    from linear_attention_token_chunked_amd import gdn

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    res, _ = bench_prefill(args.workload, gdn, torch, args.steps, args.warmup)
    traffic = measured_traffic("prefill", args.workload)
    dec = None if args.no_decode else bench_decode(gdn, torch)
    ver = None if args.no_decode else bench_verify(gdn, torch)
    epi = None if args.no_decode else bench_epilogue(gdn, torch)
    conv = None if args.no_decode else bench_short_conv(gdn, torch)
    bwd = None if args.no_decode else bench_bwd(gdn, torch)
    extra = {}
    if args.all:
        for name in ("prefill_t65536_gqa", "varlen_64"):
            r, _ = bench_prefill(name, gdn, torch, max(3, args.steps // 10), 2)
            r["pct_mfma_peak"] = round(100 * r["tflops"] / PEAK_BF16_TFLOPS, 2)
            extra[name] = r
            torch.cuda.empty_cache()
    if args.pmc_calib_mib:
        src = torch.empty(args.pmc_calib_mib << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
    line = {
        "metric": "GDN prefill Mtok/s + % MFMA peak; decode-step HBM GB/s vs peak (1 GPU)",
        "value": round(res["Mtok_s"], 3),
        "unit": "Mtok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": res["workload"], "batch": res["B"], "seq_len": res["T"], "qk_heads": res["Hqk"],
                   "v_heads": res["Hv"], "head_dim_k": res["dk"], "head_dim_v": res["dv"], "chunk": res["chunk"],
                   "state_dtype": "fp32", "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(res["tflops"], 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(res["tflops"] / PEAK_BF16_TFLOPS, 4), "traffic": traffic},
        "prefill": {k: (round(v, 4) if isinstance(v, float) else v) for k, v in res.items()},
        "decode": dec,
        "verify": ver,
        "epilogue": epi,
        "short_conv": conv,
        "bwd": bwd,
        "cpu_baseline": cpu,
    }
    if extra:
        line["extra"] = extra
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""GDN token-mixer benchmark on one MI355X.

One step = one gdn_fwd_chunked call (chunk-local gates, UT transform, W/U,
masked products, state scan, outputs and final states) over the largest
prefill workload: 64 packed sequences of lognormal length (210,119 tokens at
seed 0), 16 q/k heads shared by 32 value heads, dk = dv = 128, bf16 in, fp32
states ("varlen_64").  ``value`` is that prefill's throughput in Mtok/s with
inputs resident in HBM.  The same JSON line also carries
  roofline      the prefill call's achieved algorithmic TFLOP/s against the
                2.5 PFLOP/s dense bf16 matrix-core peak, timed with HIP events
                on the launch stream around the K back-to-back launches;
  prefill       the headline's details: cold first call, per-launch p10/p90,
                the time with a 512 MB scratch write between launches (caches
                flushed), and the spread over three repeats of the K launches;
  prefill_other the two other bf16 prefill workloads (4 x 4096 tokens x 16
                heads; one 65,536-token row with 16 q/k / 32 value heads),
                each with its own roofline, measured the same way;
  decode        64 consecutive gdn_decode_step calls on 256 sequences x 32 value
                heads (512 MiB fp32 state): algorithmic GB/s against 8 TB/s;
  verify        gdn_decode_verify, 4 drafted tokens per sequence from the same
                kind of live state: algorithmic GB/s against 8 TB/s;
  epilogue      gdn_output_norm_gate over an output of the headline's tokens (210,119 tokens x 32
                value heads): GB/s against 8 TB/s;
  short_conv    gdn_short_conv with L2 norm over a q of the headline's tokens and sequence starts
                (16 heads): GB/s against 8 TB/s;
  bwd           gdn_bwd_chunked (all gradients) over the 4 x 4096 x 16-head prefill:
                algorithmic GB/s against 8 TB/s (its 197 flops per algorithmic
                byte sit below the chip's ridge), and its dense-tile TFLOP/s;
  cpu_baseline  the fp64 oracle on the host cores over the whole headline
                workload, and the relative L2 error of the GPU's o and final
                states against it (rel_l2_o, rel_l2_state).
Inputs are seeded synthetic tensors (linear_attention_token_chunked_amd.inputs).
Every timed loop starts after W untimed steps and at least --warm-seconds of
untimed load, so that it sees the GPU at its steady clocks.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--warm-seconds S] [--no-cpu-baseline]
                       [--workload NAME] [--no-others] [--no-decode]
"""

from __future__ import annotations

import argparse
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
EPILOGUE_WORKLOAD = "epilogue_varlen_64"
SHORT_CONV_WORKLOAD = "short_conv_q_varlen_64"


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


def measured_traffic(family, workload):
    """HBM bytes per call from committed rocprofv3 FETCH_SIZE/WRITE_SIZE runs, or None when they
    are missing or were taken on different kernel sources."""
    from linear_attention_token_chunked_amd.rocprof_summary import sources_hash

    try:
        rec = json.load(open(TRAFFIC_FILE))[f"{family}@{workload}"]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("sources_sha256_16") != sources_hash(family):
        return None
    return rec.get("bytes_per_call")


# ------------------------------------------------------------------ CPU baseline
def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(pool, workers, inp, o, fin):
    """The fp64 oracle over every (sequence, query/key head) piece of the workload on `workers`
    forked processes (created before this process touched the GPU), timed as a whole, and the
    relative L2 error of the GPU result (o, fin) against it."""
    from oracle.parallel import prefill_errors

    err, dt, tokens = prefill_errors(pool, inp, o, fin)
    s = err.summary()
    return {"value": round(tokens / dt / 1e6, 5), "unit": "Mtok/s", "cores": workers, "kind": "oracle",
            "sample": f"whole workload: {tokens} tokens, all {s['units']} (sequence, value head) units of the fp64 "
                      f"token recurrence, one piece per (sequence, q/k head), {dt:.1f} s wall on {workers} processes",
            "seconds": round(dt, 2), "cpu_model": cpu_model(), "affinity_cpus": len(os.sched_getaffinity(0)),
            "rel_l2_o": s["rel_l2_o"], "rel_l2_state": s["rel_l2_state"],
            "worst_unit_rel_l2_o": s["worst_unit_o"][1], "worst_unit_rel_l2_state": s["worst_unit_state"][1],
            "finite": s["finite"]}


# ------------------------------------------------------------------ GPU timing
WARM_SECONDS = 1.0  # set from --warm-seconds


def time_launches(fn, steps, warmup, torch, warm_seconds=None):
    """Run fn() warmup times, and on for at least WARM_SECONDS of wall time in all, then time
    exactly `steps` calls back to back: wall clock around the whole loop (synchronised on both
    sides) and one pair of HIP events on the launch stream around it.  Returns the wall time
    (s), the event time per launch (ms) and, from a second loop of `steps` calls with events
    around every launch, the sorted per-launch times (ms).  (Events between launches cost the
    stream a few microseconds each, so the first loop has none.)
    The GPU raises its clocks only after some hundreds of milliseconds of sustained load;
    without the timed warm-up the first launches of a fresh process run up to 15 % slower
    than the steady state."""
    warm_seconds = WARM_SECONDS if warm_seconds is None else warm_seconds
    t0 = time.perf_counter()
    n = 0
    while n < warmup or time.perf_counter() - t0 < warm_seconds:
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


def prefill_tri_flops_per_token(Hqk, Hv, dk, dv, C):
    """Triangle-aware count: the products with a masked or triangular factor (K K^T, Q K^T, T [K|V],
    P U) counted at half their dense-tile flops."""
    return Hqk * (2 * C * dk) + Hv * (C * (dk + dv) + C * dv + 6 * dk * dv)


FLUSH_BYTES = 512 << 20  # scratch written between launches for the cache-flushed time (L2s and the 256 MB MALL)


def bench_prefill(name, gdn, torch, steps, warmup, keep=False, repeats=3, flushed=10):
    """Time gdn_fwd_chunked on one prefill workload: a cold first call; `steps` back-to-back launches
    after the warm-up (the official loop) and two more such loops for the run-to-run spread;
    per-launch p10/p90; and `flushed` launches each after a 512 MB scratch write (median)."""
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
    spread = [kern_ms]
    for _ in range(repeats - 1):
        spread.append(time_launches(step, steps, 0, torch, warm_seconds=0.0)[1])
    scratch = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
    fl = []
    for _ in range(flushed):
        scratch.fill_(1)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        step()
        e1.record()
        torch.cuda.synchronize()
        fl.append(e0.elapsed_time(e1))
    del scratch
    fl.sort()
    tokens = B * T
    flops = prefill_flops_per_token(Hqk, Hv, dk, dv, w.chunk) * tokens
    flops_tri = prefill_tri_flops_per_token(Hqk, Hv, dk, dv, w.chunk) * tokens
    nbytes = prefill_bytes(tokens, N, Hqk, Hv, dk, dv, dev["q"].element_size(), dev["initial_state"] is not None,
                           True)
    tflops = flops / (kern_ms * 1e-3) / 1e12
    res = {
        "workload": name, "tokens": tokens, "B": B, "T": T, "num_seqs": N, "Hqk": Hqk, "Hv": Hv, "dk": dk, "dv": dv,
        "chunk": w.chunk, "ms_per_step": wall / steps * 1e3, "kernel_ms_mean": kern_ms,
        "kernel_ms_p10": per[len(per) // 10], "kernel_ms_median": per[len(per) // 2],
        "kernel_ms_p90": per[(len(per) * 9) // 10], "cold_ms": cold_ms,
        "repeats_kernel_ms": [round(x, 4) for x in spread],
        "repeat_spread_pct": round(100 * (max(spread) - min(spread)) / min(spread), 2),
        "flushed_kernel_ms_median": fl[len(fl) // 2],
        "Mtok_s": tokens / (wall / steps) / 1e6, "flops_per_launch": flops, "flops_tri_per_launch": flops_tri,
        "bytes_per_launch": nbytes, "tflops": tflops, "tflops_tri": flops_tri / (kern_ms * 1e-3) / 1e12,
        "pct_mfma_peak": 100 * tflops / PEAK_BF16_TFLOPS,
        "hbm_gbps": nbytes / (kern_ms * 1e-3) / 1e9, "pct_hbm_peak": 100 * nbytes / (kern_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / PEAK_BF16_TFLOPS, 4), "traffic": measured_traffic("prefill", name)},
    }
    res = {k: (round(v, 4) if isinstance(v, float) else v) for k, v in res.items()}
    kept = None
    if keep:
        torch.cuda.synchronize()
        kept = (inp, out.cpu(), fin.cpu())
    del dev, out, fin, ws
    torch.cuda.empty_cache()
    return res, kept


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


def headline_lengths():
    """The packed sequence lengths of the headline workload (its inputs' first draw at seed 0)."""
    import numpy as np

    from linear_attention_token_chunked_amd.inputs import WORKLOADS, packed_lengths

    return packed_lengths(np.random.default_rng(0), WORKLOADS["varlen_64"].num_packed)


def gpu_normal(torch, shape, dtype, seed, scale=1.0):
    """Seeded N(0, scale^2) draws made on the GPU (tensors too large to draw on the host quickly)."""
    gen = torch.Generator(device="cuda").manual_seed(seed)
    x = torch.randn(shape, generator=gen, device="cuda", dtype=dtype)
    return x.mul_(scale) if scale != 1.0 else x


def bench_epilogue(gdn, torch, steps=20):
    """Output epilogue (zero-centred RMSNorm + sigmoid gate) over an output of the headline's tokens:
    o, z ~ N(0, 1) [tokens x 32 value heads, 128] bf16, weight ~ 0.1 N(0, 1)."""
    tokens, hv, dv = int(headline_lengths().sum()), 32, 128
    rows = tokens * hv
    dev = {"o": gpu_normal(torch, (rows, dv), torch.bfloat16, 11), "z": gpu_normal(torch, (rows, dv), torch.bfloat16, 12),
           "w": gpu_normal(torch, (dv,), torch.float32, 13, 0.1)}
    y = torch.empty_like(dev["o"])

    def step():
        gdn.output_norm_gate(dev["o"], dev["z"], dev["w"], out=y)

    wall, mean_ms, per = time_launches(step, steps, 5, torch)
    us = mean_ms * 1e3
    nbytes = 3 * rows * dv * dev["o"].element_size() + dv * 4
    gbps = nbytes / (us * 1e-6) / 1e9
    return {
        "workload": EPILOGUE_WORKLOAD, "what": f"output of the headline's tokens ({rows} rows x 128, bf16)",
        "rows": rows,
        "dv": dv, "us_per_call_mean": us, "bytes_per_call": nbytes, "GBps": gbps,
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(gbps / PEAK_HBM_GBPS, 4),
                     "traffic": measured_traffic("epilogue", EPILOGUE_WORKLOAD)},
    }


def bench_short_conv(gdn, torch, steps=20):
    """Pre-mixer short convolution + per-head L2 norm over a q of the headline's tokens, restarting at
    its sequence starts: x ~ N(0, 1) [1, tokens, 16, 128] bf16, taps ~ N(0, 1) / 2."""
    import numpy as np

    lengths = headline_lengths()
    T, H, hd = int(lengths.sum()), 16, 128
    x = gpu_normal(torch, (1, T, H, hd), torch.bfloat16, 21)
    w = gpu_normal(torch, (H * hd, 4), torch.float32, 22, 0.5)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32, device="cuda")
    y = torch.empty_like(x)

    def step():
        gdn.short_conv(x, w, cu_seqlens=cu, l2norm=True, out=y)

    wall, mean_ms, per = time_launches(step, steps, 5, torch)
    us = mean_ms * 1e3
    nbytes = 2 * x.numel() * x.element_size() + w.numel() * 4 + cu.numel() * 4
    gbps = nbytes / (us * 1e-6) / 1e9
    return {
        "workload": SHORT_CONV_WORKLOAD,
        "what": f"q of the headline's tokens ({T} tokens, 64 sequences, 16 heads x 128, bf16), width 4, L2 norm",
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
    # 198 flops per algorithmic byte, below the chip's 312 (2.5 PFLOP/s over 8 TB/s): the HBM roof is the lower one
    return {
        "workload": w.name, "tokens": tokens, "ms_per_call_mean": mean_ms, "ms_per_call_median": per[len(per) // 2],
        "Mtok_s": tokens / (mean_ms * 1e-3) / 1e6, "flops_per_call": flops, "tflops": tflops,
        "mfma_frac": round(tflops / PEAK_BF16_TFLOPS, 4), "bytes_per_call": nbytes,
        "kernels": "saving prefill, state-gradient scan, local gradients (one call = all three)",
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(gbps / PEAK_HBM_GBPS, 4),
                     "traffic": measured_traffic("bwd", w.name)},
    }


OTHER_PREFILL = ("prefill_b4_t4096", "prefill_t65536_gqa")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--warm-seconds", type=float, default=1.0,
                    help="keep warming up (untimed) for at least this long per workload")
    ap.add_argument("--workload", default="varlen_64", help="the headline prefill workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode, verify, epilogue, convolution "
                                                               "and backward legs")
    ap.add_argument("--no-others", action="store_true", help="skip the other prefill workloads")
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

    pool = workers = None
    if not args.no_cpu_baseline:
        # forked before this process touches the GPU; the oracle runs on it after the GPU legs
        from oracle.parallel import host_workers, make_pool

        workers = host_workers()
        pool = make_pool(workers)

    from linear_attention_token_chunked_amd import gdn

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    print(f"bench: prefill {args.workload}", file=sys.stderr, flush=True)
    res, kept = bench_prefill(args.workload, gdn, torch, args.steps, args.warmup, keep=pool is not None)
    others = {}
    if not args.no_others:
        for name in OTHER_PREFILL:
            if name == args.workload:
                continue
            print(f"bench: prefill {name}", file=sys.stderr, flush=True)
            others[name], _ = bench_prefill(name, gdn, torch, args.steps, args.warmup)
    legs = {}
    if not args.no_decode:
        for leg, fn in (("decode", bench_decode), ("verify", bench_verify), ("epilogue", bench_epilogue),
                        ("short_conv", bench_short_conv), ("bwd", bench_bwd)):
            print(f"bench: {leg}", file=sys.stderr, flush=True)
            legs[leg] = fn(gdn, torch)
            torch.cuda.empty_cache()
    if args.pmc_calib_mib:
        src = torch.empty(args.pmc_calib_mib << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
    cpu = None
    if pool is not None:
        print("bench: fp64 oracle on the host over the headline workload", file=sys.stderr, flush=True)
        inp, o_host, fin_host = kept
        cpu = cpu_baseline(pool, workers, inp, o_host, fin_host)
        pool.terminate()
        pool.join()
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
        "config": {"workload": res["workload"], "batch": res["B"], "seq_len": res["T"], "num_seqs": res["num_seqs"],
                   "qk_heads": res["Hqk"], "v_heads": res["Hv"], "head_dim_k": res["dk"], "head_dim_v": res["dv"],
                   "chunk": res["chunk"], "state_dtype": "fp32", "parallelism": "single GPU"},
        "roofline": res["roofline"],
        "rel_l2_o": cpu["rel_l2_o"] if cpu else None,
        "rel_l2_state": cpu["rel_l2_state"] if cpu else None,
        "prefill": {k: v for k, v in res.items() if k != "roofline"},
        "prefill_other": others or None,
        **{k: legs.get(k) for k in ("decode", "verify", "epilogue", "short_conv", "bwd")},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

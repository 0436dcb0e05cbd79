"""Seeded synthetic inputs for the GDN token mixer.

This module only draws random numbers and shapes them; it holds none of the
mixer's arithmetic.  It is the one module that both the fp64 oracle's tests and
the HIP path's tests and bench use, so that both sides see identical inputs.

Recipe (the same for every workload; seed 0 unless a caller overrides it):
  * q, k ~ N(0, 1), then L2-normalised over the head dimension per (token,
    query/key head), in float64 with no epsilon, then cast;
  * v ~ N(0, 1);
  * beta = sigmoid(z), z ~ N(0, 1), float32;
  * g = log(alpha) = -gate_scale * softplus(z'), z' ~ N(0, 1), gate_scale 0.1,
    float32 (softplus computed as logaddexp(0, z'));
  * initial states ~ N(0, 0.02^2) (standard deviation 0.02), float32;
  * packed variable-length batches draw lengths L_i = clip(rint(exp(ln 2048 +
    z_i)), 16, 32768) with z_i ~ N(0, 1).
All values are drawn in float64 by ``numpy.random.default_rng(seed)`` in the
fixed order: lengths (packed only), q, k, v, beta logits, gate logits, initial
state.  bf16 tensors are produced float64 -> float32 -> bfloat16, each step
rounding to nearest even.  Tensors are returned on the CPU.
"""

from __future__ import annotations

import dataclasses

import numpy as np
import torch

_TORCH_DTYPE = {"fp32": torch.float32, "bf16": torch.bfloat16}


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape of one synthetic workload."""

    name: str
    kind: str  # "prefill", "decode" or "verify"
    dtype: str  # "fp32" or "bf16" for q, k, v, o
    Hqk: int
    Hv: int
    dk: int
    dv: int
    chunk: int = 64
    B: int = 1  # prefill batch rows (1 for packed input)
    T: int = 0  # prefill tokens per row
    init_state: bool = False
    num_packed: int = 0  # > 0: packed variable-length batch of this many sequences
    N: int = 0  # decode: independent sequences
    steps: int = 0  # decode: consecutive single-token steps; verify: tokens per sequence


WORKLOADS = {
    # tiny fp32 prefill, parity only
    "tiny_fp32": Workload("tiny_fp32", "prefill", "fp32", Hqk=2, Hv=2, dk=64, dv=64, B=1, T=256),
    # batch of 4 x 4096 tokens, 16 heads, bf16
    "prefill_b4_t4096": Workload("prefill_b4_t4096", "prefill", "bf16", Hqk=16, Hv=16, dk=128, dv=128,
                                 B=4, T=4096),
    # one 65536-token sequence, 16 q/k heads shared by 32 v heads, given initial state
    "prefill_t65536_gqa": Workload("prefill_t65536_gqa", "prefill", "bf16", Hqk=16, Hv=32, dk=128, dv=128,
                                   B=1, T=65536, init_state=True),
    # 256 sequences x 32 v heads, 64 single-token steps on a 512 MiB fp32 state
    "decode_n256": Workload("decode_n256", "decode", "bf16", Hqk=16, Hv=32, dk=128, dv=128, N=256, steps=64,
                            init_state=True),
    # multi-token verify: 256 sequences x 32 v heads, 4 drafted tokens each, from a 512 MiB live state
    "verify_n256_t4": Workload("verify_n256_t4", "verify", "bf16", Hqk=16, Hv=32, dk=128, dv=128, N=256, steps=4,
                               init_state=True),
    # 64 packed sequences of lognormal length, per-sequence initial states
    "varlen_64": Workload("varlen_64", "prefill", "bf16", Hqk=16, Hv=32, dk=128, dv=128, num_packed=64,
                          init_state=True),
}


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _cast(x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(_TORCH_DTYPE[dtype]) if dtype != "fp32" else t


def packed_lengths(rng, n):
    """Lengths of a packed batch: clip(rint(exp(ln 2048 + z)), 16, 32768)."""
    z = rng.standard_normal(n)
    return np.clip(np.rint(np.exp(np.log(2048.0) + z)), 16, 32768).astype(np.int64)


def make_prefill(B, T, Hqk, Hv, dk, dv, dtype="bf16", init_state=False, lengths=None, seed=0,
                 gate_scale=0.1, num_packed=0):
    """Draw one prefill batch.

    ``lengths`` (explicit) or ``num_packed`` (drawn lognormal) selects a packed
    batch: then B = 1, T = sum(lengths) and cu_seqlens is returned.
    Returns a dict of CPU tensors: q, k [B, T, Hqk, dk]; v [B, T, Hv, dv];
    g, beta [B, T, Hv] fp32; initial_state [N, Hv, dk, dv] fp32 or None;
    cu_seqlens int32 [N + 1] or None.
    """
    rng = np.random.default_rng(seed)
    cu = None
    if num_packed and lengths is None:
        lengths = packed_lengths(rng, num_packed)
    if lengths is not None:
        lengths = np.asarray(lengths, dtype=np.int64)
        B, T = 1, int(lengths.sum())
        cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    N = len(lengths) if lengths is not None else B
    q = _unit(rng.standard_normal((B, T, Hqk, dk)))
    k = _unit(rng.standard_normal((B, T, Hqk, dk)))
    v = rng.standard_normal((B, T, Hv, dv))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, Hv))))
    g = -gate_scale * np.logaddexp(0.0, rng.standard_normal((B, T, Hv)))
    s0 = 0.02 * rng.standard_normal((N, Hv, dk, dv)) if init_state else None
    out = {
        "q": _cast(q, dtype),
        "k": _cast(k, dtype),
        "v": _cast(v, dtype),
        "g": _cast(g, "fp32"),
        "beta": _cast(beta, "fp32"),
        "initial_state": _cast(s0, "fp32") if s0 is not None else None,
        "cu_seqlens": torch.from_numpy(cu) if cu is not None else None,
    }
    return out


def make_decode(N, Hqk, Hv, dk, dv, steps, dtype="bf16", seed=0, gate_scale=0.1):
    """Draw a decode run: per-step q, k [steps, N, Hqk, dk], v [steps, N, Hv, dv],
    g, beta [steps, N, Hv] and the initial state [N, Hv, dk, dv] fp32."""
    rng = np.random.default_rng(seed)
    q = _unit(rng.standard_normal((steps, N, Hqk, dk)))
    k = _unit(rng.standard_normal((steps, N, Hqk, dk)))
    v = rng.standard_normal((steps, N, Hv, dv))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((steps, N, Hv))))
    g = -gate_scale * np.logaddexp(0.0, rng.standard_normal((steps, N, Hv)))
    s0 = 0.02 * rng.standard_normal((N, Hv, dk, dv))
    return {
        "q": _cast(q, dtype),
        "k": _cast(k, dtype),
        "v": _cast(v, dtype),
        "g": _cast(g, "fp32"),
        "beta": _cast(beta, "fp32"),
        "state": _cast(s0, "fp32"),
    }


def make_verify(N, Tv, Hqk, Hv, dk, dv, dtype="bf16", seed=0, gate_scale=0.1):
    """Draw a multi-token verify call: the decode draws of make_decode for Tv steps,
    laid out per sequence: q, k [N, Tv, Hqk, dk], v [N, Tv, Hv, dv], g, beta [N, Tv, Hv],
    and the live state [N, Hv, dk, dv] fp32."""
    d = make_decode(N, Hqk, Hv, dk, dv, Tv, dtype, seed=seed, gate_scale=gate_scale)
    out = {name: d[name].transpose(0, 1).contiguous() for name in ("q", "k", "v", "g", "beta")}
    out["state"] = d["state"]
    return out


def make_epilogue(rows, dv, dtype="bf16", seed=0):
    """Draw output-epilogue inputs: mixer outputs o and gate pre-activations z [rows, dv]
    ~ N(0, 1), and the zero-centred norm weight w [dv] ~ 0.1 N(0, 1) fp32."""
    rng = np.random.default_rng(seed)
    return {
        "o": _cast(rng.standard_normal((rows, dv)), dtype),
        "z": _cast(rng.standard_normal((rows, dv)), dtype),
        "w": _cast(0.1 * rng.standard_normal(dv), "fp32"),
    }


def make_conv(B, T, heads, head_dim, dtype="bf16", seed=0, num_packed=0):
    """Draw short-convolution inputs: pre-convolution activations x [B, T, heads, head_dim]
    ~ N(0, 1), taps [heads * head_dim, 4] ~ N(0, 1) / 2 fp32, and (num_packed > 0, B = 1)
    cu_seqlens for that many sequences of lognormal length over the T tokens."""
    rng = np.random.default_rng(seed)
    out = {
        "x": _cast(rng.standard_normal((B, T, heads, head_dim)), dtype),
        "w": _cast(0.5 * rng.standard_normal((heads * head_dim, 4)), "fp32"),
        "cu_seqlens": None,
    }
    if num_packed:
        cuts = np.sort(rng.choice(np.arange(1, T), size=num_packed - 1, replace=False))
        out["cu_seqlens"] = torch.from_numpy(np.concatenate([[0], cuts, [T]]).astype(np.int32))
    return out


def make_cotangents(B, T, Hv, dv, N, dk, dtype="bf16", seed=0, final=True):
    """Draw the incoming gradients of a prefill's backward pass: d_o [B, T, Hv, dv] ~ N(0, 1)
    in the activations' dtype, and d_final [N, Hv, dk, dv] ~ 0.1 N(0, 1) fp32 (or None)."""
    rng = np.random.default_rng(seed + 7919)
    return {
        "d_o": _cast(rng.standard_normal((B, T, Hv, dv)), dtype),
        "d_final": _cast(0.1 * rng.standard_normal((N, Hv, dk, dv)), "fp32") if final else None,
    }


def make_workload(w: Workload, seed=0, gate_scale=0.1):
    """Inputs for one named workload (see WORKLOADS)."""
    if w.kind == "verify":
        return make_verify(w.N, w.steps, w.Hqk, w.Hv, w.dk, w.dv, w.dtype, seed=seed, gate_scale=gate_scale)
    if w.kind == "decode":
        return make_decode(w.N, w.Hqk, w.Hv, w.dk, w.dv, w.steps, w.dtype, seed=seed, gate_scale=gate_scale)
    return make_prefill(w.B, w.T, w.Hqk, w.Hv, w.dk, w.dv, w.dtype, init_state=w.init_state, seed=seed,
                        gate_scale=gate_scale, num_packed=w.num_packed)

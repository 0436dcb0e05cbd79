"""Parallel driver of the fp64 oracle over independent units, with error norms.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
use it.  It holds none of the mixer's arithmetic: every result comes from
``recurrent`` and ``decode_step`` in ``gdn_oracle.py`` and ``recurrent_grads`` in
``backward.py``; this module only cuts a
workload into independent pieces, runs the oracle on them in forked worker
processes and measures how far a candidate result is from the oracle's.

Independence (the definition itself, reading R6 and R9): every sequence and
every value head is its own recurrence, and the value heads that share a
query/key head read the same q and k.  So a piece is one (sequence, query/key
head) pair with all of its value heads; for decode, one sequence with all of
its heads over every step.

Error measure (reading R17): relative L2 over a whole tensor is
sqrt(sum (x - y)^2 / sum y^2) with y the oracle, accumulated piece by piece in
float64; the same ratio is also kept per (sequence, value head) unit.

The pool must be created before the calling process initialises the GPU: the
workers are forked from it.  Inputs and candidate results travel to the workers
as raw bf16 bits or float32 values (both upcast exactly to float64 there).
"""

from __future__ import annotations

import multiprocessing as mp
import os
import time

import numpy as np

from .backward import recurrent_grads
from .gdn_oracle import decode_step, recurrent

__all__ = ["host_workers", "grad_workers", "make_pool", "prefill_errors", "decode_errors", "bwd_errors", "Errors", "GRADS"]


def host_workers():
    """Worker count: the CPUs this process may run on, limited to the CPU share the host
    declares through OMP_NUM_THREADS when it sets one."""
    n = len(os.sched_getaffinity(0))
    share = os.environ.get("OMP_NUM_THREADS", "")
    if share.isdigit() and int(share) > 0:
        n = min(n, int(share))
    return max(1, n)


def grad_workers():
    """Worker count for pieces that run the autograd oracle (recurrent_grads): its first backward
    pass makes torch ask the GPU runtime how many devices there are, which opens the GPU in that
    process; at most 14, so that with the caller such a pool stays within the 16 processes a GPU
    host admits with the GPU open."""
    return max(1, min(14, host_workers() - 2))


def _worker_init():
    # one BLAS thread per worker: the pieces are the parallelism
    try:
        from threadpoolctl import threadpool_limits

        threadpool_limits(1)
    except ImportError:
        pass


def make_pool(workers=None):
    """A fork-context pool.  Call it before this process makes its first GPU call."""
    return mp.get_context("fork").Pool(workers or host_workers(), initializer=_worker_init)


# ---------------------------------------------------------------- exact transport of bf16 / fp32 data
def _pack(t):
    """A CPU torch tensor as (kind, numpy array): bf16 as its raw 16-bit patterns, fp32 as is."""
    import torch

    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return ("bf16", t.view(torch.int16).numpy())
    return ("f32", t.to(torch.float32).numpy())


def _unpack(p):
    kind, a = p
    if kind == "bf16":
        return (a.astype(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


class Errors:
    """Sums of squares of (candidate - oracle) and of the oracle, whole-tensor and per unit, for each
    named result (o and the final state; or the gradients)."""

    def __init__(self, keys=("o", "state")):
        self.keys = tuple(keys)
        self.d = {key: 0.0 for key in self.keys}
        self.r = {key: 0.0 for key in self.keys}
        self.unit = {key: {} for key in self.keys}  # unit -> relative L2
        self.finite = True
        self.units = 0

    def add(self, res):
        for key in self.keys:
            for unit, (d, r) in res[key].items():
                self.d[key] += d
                self.r[key] += r
                self.unit[key][unit] = np.sqrt(d / r) if r > 0 else np.sqrt(d)
        self.finite &= res["finite"]
        self.units += len(res[self.keys[0]])

    def rel(self, key):
        return float(np.sqrt(self.d[key] / self.r[key])) if self.r[key] > 0 else float(np.sqrt(self.d[key]))

    def worst(self, key):
        if not self.unit[key]:
            return (None, 0.0)
        u = max(self.unit[key], key=self.unit[key].get)
        return (u, float(self.unit[key][u]))

    def summary(self):
        (uo, wo), (us, ws) = self.worst("o"), self.worst("state")
        return {"rel_l2_o": self.rel("o"), "rel_l2_state": self.rel("state"), "units": self.units,
                "worst_unit_o": [uo, wo], "worst_unit_state": [us, ws], "finite": bool(self.finite)}


def _sq(x, y):
    e = x - y
    return float(np.sum(e * e)), float(np.sum(y * y))


# ---------------------------------------------------------------- prefill
def _prefill_piece(args):
    """Worker: the oracle on one (sequence, query/key head) piece; error sums against the candidate."""
    n, heads, q, k, v, g, beta, s0, o_c, s_c, scale = args
    q, k, v, o_c = (_unpack(x) for x in (q, k, v, o_c))
    g, beta = _unpack(g), _unpack(beta)
    s0 = _unpack(s0) if s0 is not None else None
    s_c = _unpack(s_c) if s_c is not None else None
    # [L, d] / [L, rep, d] -> the oracle's [1, L, H, d] layout with one query/key head and rep value heads
    ro, rf = recurrent(q[None, :, None], k[None, :, None], v[None], g[None], beta[None],
                       initial_state=None if s0 is None else s0[None], scale=scale)
    res = {"o": {}, "state": {}, "finite": bool(np.all(np.isfinite(o_c)))}
    for i, h in enumerate(heads):
        res["o"][(n, h)] = _sq(o_c[:, i], ro[0, :, i])
        if s_c is not None:
            res["finite"] &= bool(np.all(np.isfinite(s_c[i])))
            res["state"][(n, h)] = _sq(s_c[i], rf[0, i])
    return res


def prefill_errors(pool, inp, o, final_state, scale=1.0):
    """Whole-workload error of a prefill result against the oracle's token recurrence.

    ``inp``: the CPU input dict (q, k [B, T, Hqk, dk]; v [B, T, Hv, dv]; g, beta;
    initial_state or None; cu_seqlens or None); ``o``, ``final_state``: the candidate
    result (CPU or GPU tensors; final_state may be None).  Returns (Errors, wall seconds
    of the oracle over every piece, tokens)."""
    q, k, v, g, beta = (inp[x] for x in ("q", "k", "v", "g", "beta"))
    S0, cu = inp.get("initial_state"), inp.get("cu_seqlens")
    B, T, Hqk, _ = q.shape
    Hv = v.shape[2]
    rep = Hv // Hqk
    o = o.detach().cpu()
    fs = final_state.detach().cpu() if final_state is not None else None
    if cu is not None:
        cu = [int(x) for x in cu]
        seqs = [(0, cu[i], cu[i + 1]) for i in range(len(cu) - 1)]
    else:
        seqs = [(b, 0, T) for b in range(B)]

    def pieces():
        order = sorted(range(len(seqs)), key=lambda i: seqs[i][1] - seqs[i][2])  # longest first
        for n in order:
            b, s, e = seqs[n]
            for hq in range(Hqk):
                hs = slice(hq * rep, (hq + 1) * rep)
                yield (n, list(range(hq * rep, (hq + 1) * rep)), _pack(q[b, s:e, hq]), _pack(k[b, s:e, hq]),
                       _pack(v[b, s:e, hs]), _pack(g[b, s:e, hs]), _pack(beta[b, s:e, hs]),
                       _pack(S0[n, hs]) if S0 is not None else None, _pack(o[b, s:e, hs]),
                       _pack(fs[n, hs]) if fs is not None else None, scale)

    err = Errors()
    t0 = time.perf_counter()
    for res in pool.imap_unordered(_prefill_piece, pieces(), chunksize=1):
        err.add(res)
    dt = time.perf_counter() - t0
    return err, dt, B * T


# ---------------------------------------------------------------- decode
def _decode_piece(args):
    """Worker: ``steps`` oracle decode steps of one sequence, every head; error sums of o (all steps)
    and of the state after the last step."""
    n, q, k, v, g, beta, s0, o_c, s_c, scale = args
    q, k, v, g, beta, s0, o_c, s_c = (_unpack(x) for x in (q, k, v, g, beta, s0, o_c, s_c))
    state = s0[None]
    steps, Hv = v.shape[0], v.shape[1]
    ro = np.zeros_like(o_c)
    for t in range(steps):
        o_t, state = decode_step(q[t][None], k[t][None], v[t][None], g[t][None], beta[t][None], state, scale=scale)
        ro[t] = o_t[0]
    res = {"o": {}, "state": {}, "finite": bool(np.all(np.isfinite(o_c)) and np.all(np.isfinite(s_c)))}
    for h in range(Hv):
        res["o"][(n, h)] = _sq(o_c[:, h], ro[:, h])
        res["state"][(n, h)] = _sq(s_c[h], state[0, h])
    return res


def decode_errors(pool, inp, o_steps, final_state, scale=1.0):
    """Whole-workload error of ``steps`` consecutive decode steps against the oracle's decode_step.

    ``inp``: make_decode's dict (q, k [steps, N, Hqk, dk]; v [steps, N, Hv, dv]; g, beta
    [steps, N, Hv]; state [N, Hv, dk, dv] before the first step); ``o_steps`` [steps, N, Hv, dv]
    and ``final_state`` [N, Hv, dk, dv]: the candidate.  Returns (Errors, wall seconds)."""
    q, k, v, g, beta, s0 = (inp[x] for x in ("q", "k", "v", "g", "beta", "state"))
    o_steps = o_steps.detach().cpu()
    fs = final_state.detach().cpu()
    N = s0.shape[0]

    def pieces():
        for n in range(N):
            yield (n, _pack(q[:, n]), _pack(k[:, n]), _pack(v[:, n]), _pack(g[:, n]), _pack(beta[:, n]),
                   _pack(s0[n]), _pack(o_steps[:, n]), _pack(fs[n]), scale)

    err = Errors()
    t0 = time.perf_counter()
    for res in pool.imap_unordered(_decode_piece, pieces(), chunksize=4):
        err.add(res)
    return err, time.perf_counter() - t0


# ---------------------------------------------------------------- backward
GRADS = ("dq", "dk", "dv", "dg", "dbeta", "d_initial_state")


def _bwd_piece(args):
    """Worker: the autograd oracle's gradients of one (sequence, query/key head) piece; error sums
    against the candidate's.  dq and dk are one unit per (sequence, query/key head) (summed over its
    value heads); the other gradients one unit per (sequence, value head)."""
    import torch

    torch.set_num_threads(1)
    n, hq, heads, q, k, v, g, beta, d_o, s0, dfin, cand, scale = args
    q, k, v, g, beta, d_o = (_unpack(x) for x in (q, k, v, g, beta, d_o))
    s0 = _unpack(s0) if s0 is not None else None
    dfin = _unpack(dfin) if dfin is not None else None
    cand = {key: (_unpack(x) if x is not None else None) for key, x in cand.items()}
    ref = recurrent_grads(q[None, :, None], k[None, :, None], v[None], g[None], beta[None], d_o[None],
                          initial_state=None if s0 is None else s0[None],
                          d_final=None if dfin is None else dfin[None], scale=scale)
    res = {key: {} for key in GRADS}
    res["finite"] = all(bool(np.all(np.isfinite(x))) for x in cand.values() if x is not None)
    res["dq"][(n, hq)] = _sq(cand["dq"], ref["dq"][0, :, 0])
    res["dk"][(n, hq)] = _sq(cand["dk"], ref["dk"][0, :, 0])
    for i, h in enumerate(heads):
        for key in ("dv", "dg", "dbeta"):
            res[key][(n, h)] = _sq(cand[key][:, i], ref[key][0, :, i])
        if cand["d_initial_state"] is not None:
            res["d_initial_state"][(n, h)] = _sq(cand["d_initial_state"][i], ref["d_initial_state"][0, i])
    return res


def bwd_errors(pool, inp, cot, grads, scale=1.0, progress=None):
    """Whole-workload error of a backward result against the autograd oracle (``recurrent_grads``).

    ``inp``: the forward's CPU input dict; ``cot``: d_o [B, T, Hv, dv] and d_final [N, Hv, dk, dv]
    or None; ``grads``: the candidate's dict (dq, dk, dv, dg, dbeta, d_initial_state or None);
    ``progress(done, total)``, if given, is called as pieces finish.
    Returns (Errors over GRADS, wall seconds)."""
    q, k, v, g, beta = (inp[x] for x in ("q", "k", "v", "g", "beta"))
    S0, cu = inp.get("initial_state"), inp.get("cu_seqlens")
    d_o, dfin = cot["d_o"], cot.get("d_final")
    B, T, Hqk, _ = q.shape
    Hv = v.shape[2]
    rep = Hv // Hqk
    cpu = {key: (x.detach().cpu() if x is not None else None) for key, x in grads.items()}
    if cu is not None:
        cu = [int(x) for x in cu]
        seqs = [(0, cu[i], cu[i + 1]) for i in range(len(cu) - 1)]
    else:
        seqs = [(b, 0, T) for b in range(B)]

    def pieces():
        order = sorted(range(len(seqs)), key=lambda i: seqs[i][1] - seqs[i][2])  # longest first
        for n in order:
            b, s, e = seqs[n]
            for hq in range(Hqk):
                hs = slice(hq * rep, (hq + 1) * rep)
                cand = {"dq": _pack(cpu["dq"][b, s:e, hq]), "dk": _pack(cpu["dk"][b, s:e, hq])}
                for key in ("dv", "dg", "dbeta"):
                    cand[key] = _pack(cpu[key][b, s:e, hs])
                dh0 = cpu.get("d_initial_state")
                cand["d_initial_state"] = _pack(dh0[n, hs]) if dh0 is not None else None
                yield (n, hq, list(range(hq * rep, (hq + 1) * rep)), _pack(q[b, s:e, hq]), _pack(k[b, s:e, hq]),
                       _pack(v[b, s:e, hs]), _pack(g[b, s:e, hs]), _pack(beta[b, s:e, hs]), _pack(d_o[b, s:e, hs]),
                       _pack(S0[n, hs]) if S0 is not None else None,
                       _pack(dfin[n, hs]) if dfin is not None else None, cand, scale)

    err = Errors(GRADS)
    total = len(seqs) * Hqk
    t0 = time.perf_counter()
    for done, res in enumerate(pool.imap_unordered(_bwd_piece, pieces(), chunksize=1), 1):
        err.add(res)
        if progress:
            progress(done, total)
    return err, time.perf_counter() - t0

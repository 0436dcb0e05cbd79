"""Helpers for the GPU parity tests: tolerance, error measures and per-unit oracle runs.

Tolerances (relative L2 error against the fp64 oracle, over a whole tensor and
also over every (sequence, value head) unit separately):
  fp32 inputs: 1e-5;  bf16 inputs: 2e-2.
"""

import sys

import numpy as np
import torch

from oracle import recurrent

TOL = {torch.float32: 1e-5, torch.bfloat16: 2e-2}


def flush(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def rel_l2(x, y):
    x, y = np.asarray(x, np.float64), np.asarray(y, np.float64)
    den = np.linalg.norm(y.ravel())
    num = np.linalg.norm((x - y).ravel())
    return num / den if den > 0 else num


def to_dev(d, dev="cuda"):
    return {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


def assert_close(name, got, ref, tol):
    err = rel_l2(got, ref)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    assert err <= tol, f"{name}: rel-L2 {err:.3e} > {tol:.1e}"
    return err


def unit_oracle(inp, n, h, cu=None, T=None):
    """Oracle for one (sequence n, value head h) unit of a prefill batch: returns (o [L, dv], final [dk, dv])."""
    q, k, v, g, beta = (inp[x] for x in ("q", "k", "v", "g", "beta"))
    Hqk, Hv = q.shape[2], v.shape[2]
    hq = h // (Hv // Hqk)
    if cu is not None:
        b, s, e = 0, int(cu[n]), int(cu[n + 1])
    else:
        b, s, e = n, 0, q.shape[1]
    sl = lambda t, head: t[b:b + 1, s:e, head:head + 1]
    S0 = inp.get("initial_state")
    S0 = S0[n:n + 1, h:h + 1] if S0 is not None else None
    o, fin = recurrent(sl(q, hq), sl(k, hq), sl(v, h), g[b:b + 1, s:e, h:h + 1], beta[b:b + 1, s:e, h:h + 1],
                       initial_state=S0)
    return o[0, :, 0], fin[0, 0]

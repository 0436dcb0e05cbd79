"""Helpers for the GPU parity tests: tolerance, error measures and per-unit oracle runs.

Tolerances (relative L2 error against the fp64 oracle, over a whole tensor and
also over every (sequence, value head) unit separately):
  fp32 inputs: 1e-5;  bf16 inputs: 2e-2.
"""

import sys

import numpy as np
import torch


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


def whole_check(pool, inp, o, fin, tol, label, scale=1.0):
    """Whole-workload parity of a prefill result (see oracle.parallel): relative L2 of o and of the final
    states over the whole tensors, and the worst (sequence, value head) unit, all within tol."""
    from oracle.parallel import prefill_errors

    err, secs, _ = prefill_errors(pool, inp, o, fin, scale=scale)
    s = err.summary()
    flush(f"  {label}: rel-L2 o {s['rel_l2_o']:.3e} state {s['rel_l2_state']:.3e} over {s['units']} units; "
          f"worst unit o {s['worst_unit_o'][0]} {s['worst_unit_o'][1]:.3e}, "
          f"state {s['worst_unit_state'][0]} {s['worst_unit_state'][1]:.3e} (oracle {secs:.1f} s)")
    assert s["finite"], f"{label}: non-finite values"
    assert s["rel_l2_o"] <= tol and s["rel_l2_state"] <= tol, f"{label}: whole-tensor rel-L2 above {tol}"
    assert s["worst_unit_o"][1] <= tol and s["worst_unit_state"][1] <= tol, f"{label}: a unit above {tol}"
    return s

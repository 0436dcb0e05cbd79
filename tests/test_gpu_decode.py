"""GPU parity of gdn_decode_step against the fp64 oracle (through the C ABI)."""

import numpy as np
import pytest
import torch

from oracle import decode_step as oracle_decode
from parity import TOL, assert_close, f64, flush, to_dev

from linear_attention_token_chunked_amd.inputs import WORKLOADS, make_decode

pytestmark = pytest.mark.gpu
DT = {"bf16": torch.bfloat16, "fp32": torch.float32}


@pytest.fixture(scope="module")
def gdn():
    from linear_attention_token_chunked_amd import gdn as m

    return m


@pytest.mark.parametrize("dtype,dk,dv,Hqk,Hv", [
    ("bf16", 128, 128, 2, 4),
    ("fp32", 64, 64, 1, 2),
    ("fp32", 128, 128, 2, 4),
    ("bf16", 128, 64, 2, 2),
    ("bf16", 64, 128, 1, 3),
])
def test_decode_small_matches_oracle(gdn, dtype, dk, dv, Hqk, Hv):
    flush(f"decode small {dtype} dk={dk} dv={dv} Hqk={Hqk} Hv={Hv}")
    steps, N = 6, 5
    inp = make_decode(N, Hqk, Hv, dk, dv, steps, dtype, seed=11)
    dev = to_dev(inp)
    state = dev["state"].clone()
    ref_state = f64(inp["state"])
    outs, refs = [], []
    for t in range(steps):
        o = gdn.decode_step(dev["q"][t], dev["k"][t], dev["v"][t], dev["g"][t], dev["beta"][t], state, scale=0.8)
        ro, ref_state = oracle_decode(inp["q"][t], inp["k"][t], inp["v"][t], inp["g"][t], inp["beta"][t], ref_state,
                                      scale=0.8)
        outs.append(f64(o))
        refs.append(ro)
    tol = TOL[DT[dtype]]
    assert_close("o", np.stack(outs), np.stack(refs), tol)
    assert_close("state", f64(state), ref_state, tol)


def test_decode_full_workload_sampled_units(gdn):
    """256 sequences x 32 value heads, 64 steps in place; oracle on 24 sampled units, all 64 steps."""
    w = WORKLOADS["decode_n256"]
    flush(f"decode full {w}")
    inp = make_decode(w.N, w.Hqk, w.Hv, w.dk, w.dv, w.steps, w.dtype, seed=0)
    dev = to_dev(inp)
    state = dev["state"].clone()
    outs = []
    for t in range(w.steps):
        outs.append(gdn.decode_step(dev["q"][t], dev["k"][t], dev["v"][t], dev["g"][t], dev["beta"][t], state))
    o_all = torch.stack(outs)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o_all.float()).all()) and bool(torch.isfinite(state).all())
    rng = np.random.default_rng(123)
    units = [(0, 0), (w.N - 1, w.Hv - 1)] + [(int(a), int(b)) for a, b in
                                             zip(rng.integers(0, w.N, 22), rng.integers(0, w.Hv, 22))]
    rep = w.Hv // w.Hqk
    got_o, ref_o, got_s, ref_s = [], [], [], []
    for n, h in units:
        hq = h // rep
        s = f64(inp["state"][n:n + 1, h:h + 1])
        for t in range(w.steps):
            ro, s = oracle_decode(inp["q"][t][n:n + 1, hq:hq + 1], inp["k"][t][n:n + 1, hq:hq + 1],
                                  inp["v"][t][n:n + 1, h:h + 1], inp["g"][t][n:n + 1, h:h + 1],
                                  inp["beta"][t][n:n + 1, h:h + 1], s)
            ref_o.append(ro[0, 0])
            got_o.append(f64(o_all[t, n, h]))
        ref_s.append(s[0, 0])
        got_s.append(f64(state[n, h]))
        assert_close(f"o unit {(n, h)}", np.stack(got_o[-w.steps:]), np.stack(ref_o[-w.steps:]), TOL[torch.bfloat16])
    assert_close("o sampled", np.stack(got_o), np.stack(ref_o), TOL[torch.bfloat16])
    assert_close("state sampled", np.stack(got_s), np.stack(ref_s), TOL[torch.bfloat16])

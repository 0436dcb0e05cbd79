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


def test_decode_zero_gates(gdn):
    """alpha = 0 (g = -inf) for some (sequence, head) units at some steps: their state is replaced by
    beta v k^T, exactly as the token recurrence says, and nothing becomes NaN."""
    flush("decode zero gates")
    steps, N = 4, 5
    inp = make_decode(N, 2, 4, 128, 128, steps, "bf16", seed=12)
    for t, n, h in [(0, 0, 0), (1, 2, 3), (2, 4, 1), (3, 0, 0)]:
        inp["g"][t, n, h] = -float("inf")
    dev = to_dev(inp)
    state = dev["state"].clone()
    ref_state = f64(inp["state"])
    outs, refs = [], []
    for t in range(steps):
        o = gdn.decode_step(dev["q"][t], dev["k"][t], dev["v"][t], dev["g"][t], dev["beta"][t], state)
        ro, ref_state = oracle_decode(inp["q"][t], inp["k"][t], inp["v"][t], inp["g"][t], inp["beta"][t], ref_state)
        outs.append(f64(o))
        refs.append(ro)
    got_o, got_s = np.stack(outs), f64(state)
    assert np.all(np.isfinite(got_o)) and np.all(np.isfinite(got_s))
    assert_close("o", got_o, np.stack(refs), TOL[torch.bfloat16])
    assert_close("state", got_s, ref_state, TOL[torch.bfloat16])


def test_decode_max_value_heads(gdn):
    """4096 value heads over 2048 q/k heads (the largest head count the boundary accepts), two steps: every
    output finite, and the first and last heads match the oracle (run on those heads alone)."""
    N, Hqk, Hv, steps = 2, 2048, 4096, 2
    flush(f"decode max heads N={N} Hqk={Hqk} Hv={Hv}")
    inp = make_decode(N, Hqk, Hv, 128, 128, steps, "bf16", seed=13)
    dev = to_dev(inp)
    state = dev["state"].clone()
    heads = [0, 1, 2047, 2048, 4094, 4095]
    qk = [h // (Hv // Hqk) for h in heads]
    ref_state = f64(inp["state"][:, heads])
    for t in range(steps):
        o = gdn.decode_step(dev["q"][t], dev["k"][t], dev["v"][t], dev["g"][t], dev["beta"][t], state)
        ro, ref_state = oracle_decode(inp["q"][t][:, qk], inp["k"][t][:, qk], inp["v"][t][:, heads],
                                      inp["g"][t][:, heads], inp["beta"][t][:, heads], ref_state)
        go = f64(o)
        assert np.all(np.isfinite(go))
        assert_close(f"o step {t}", go[:, heads], ro, TOL[torch.bfloat16])
    gs = f64(state)
    assert np.all(np.isfinite(gs))
    assert_close("state", gs[:, heads], ref_state, TOL[torch.bfloat16])


def test_decode_full_workload_whole_tensors(gdn, oracle_pool):
    """256 sequences x 32 value heads, 64 separate decode calls updating the 512 MiB state in place: every
    element of o at every step and of the state after step 64 against 64 oracle decode steps per sequence
    (forked host processes, one sequence each), whole tensors and every (sequence, value head) unit."""
    from oracle.parallel import decode_errors

    w = WORKLOADS["decode_n256"]
    flush(f"decode full {w.name}: drawing inputs")
    inp = make_decode(w.N, w.Hqk, w.Hv, w.dk, w.dv, w.steps, w.dtype, seed=0)
    dev = to_dev(inp)
    state = dev["state"].clone()
    outs = []
    flush("  GPU: 64 steps")
    for t in range(w.steps):
        outs.append(gdn.decode_step(dev["q"][t], dev["k"][t], dev["v"][t], dev["g"][t], dev["beta"][t], state))
    o_all = torch.stack(outs).cpu()
    fin = state.cpu()
    torch.cuda.synchronize()
    flush("  oracle on the host")
    err, secs = decode_errors(oracle_pool, inp, o_all, fin)
    s = err.summary()
    tol = TOL[torch.bfloat16]
    flush(f"  {w.name}: rel-L2 o {s['rel_l2_o']:.3e} (64 steps) state {s['rel_l2_state']:.3e} over {s['units']} "
          f"units; worst unit o {s['worst_unit_o'][0]} {s['worst_unit_o'][1]:.3e}, state "
          f"{s['worst_unit_state'][0]} {s['worst_unit_state'][1]:.3e} (oracle {secs:.1f} s)")
    assert s["finite"] and s["units"] == w.N * w.Hv
    assert s["rel_l2_o"] <= tol and s["rel_l2_state"] <= tol
    assert s["worst_unit_o"][1] <= tol and s["worst_unit_state"][1] <= tol

"""GPU parity of gdn_decode_verify (multi-token verify from a live state) against the fp64 oracle,
through the C ABI, and its agreement with repeated gdn_decode_step calls."""

import numpy as np
import pytest
import torch

from oracle import verify as oracle_verify
from parity import TOL, assert_close, f64, flush, to_dev

from linear_attention_token_chunked_amd.inputs import WORKLOADS, make_verify

pytestmark = pytest.mark.gpu
DT = {"bf16": torch.bfloat16, "fp32": torch.float32}


@pytest.fixture(scope="module")
def gdn():
    from linear_attention_token_chunked_amd import gdn as m

    return m


@pytest.mark.parametrize("dtype,Tv,dk,dv,Hqk,Hv", [
    ("bf16", 4, 128, 128, 2, 4),
    ("bf16", 1, 128, 128, 1, 2),
    ("bf16", 8, 128, 64, 2, 2),
    ("fp32", 5, 64, 64, 1, 2),
    ("fp32", 8, 128, 128, 2, 4),
    ("bf16", 2, 64, 128, 1, 3),
])
def test_verify_small_matches_oracle(gdn, dtype, Tv, dk, dv, Hqk, Hv):
    flush(f"verify small {dtype} Tv={Tv} dk={dk} dv={dv} Hqk={Hqk} Hv={Hv}")
    N = 5
    inp = make_verify(N, Tv, Hqk, Hv, dk, dv, dtype, seed=21 + Tv)
    dev = to_dev(inp)
    state = dev["state"].clone()
    states = torch.empty((N, Tv, Hv, dk, dv), dtype=torch.float32, device="cuda")
    o = gdn.decode_verify(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], state, token_states=states, scale=0.8)
    ref_o, ref_states = oracle_verify(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["state"], scale=0.8)
    tol = TOL[DT[dtype]]
    assert_close("o", f64(o), ref_o, tol)
    assert_close("token states", f64(states), ref_states, tol)
    assert_close("state in place", f64(state), ref_states[:, -1], tol)


def test_verify_zero_gates(gdn):
    """A drafted token with alpha = 0 (g = -inf) erases its unit's live state, the first drafted token included."""
    flush("verify zero gates")
    N, Tv = 5, 4
    inp = make_verify(N, Tv, 2, 4, 128, 128, "bf16", seed=22)
    for n, t, h in [(0, 0, 0), (1, 2, 3), (4, 3, 1)]:
        inp["g"][n, t, h] = -float("inf")
    dev = to_dev(inp)
    state = dev["state"].clone()
    states = torch.empty((N, Tv, 4, 128, 128), dtype=torch.float32, device="cuda")
    o = gdn.decode_verify(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], state, token_states=states)
    ref_o, ref_states = oracle_verify(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["state"])
    tol = TOL[torch.bfloat16]
    assert np.all(np.isfinite(f64(o))) and np.all(np.isfinite(f64(states)))
    assert_close("o", f64(o), ref_o, tol)
    assert_close("token states", f64(states), ref_states, tol)


def test_verify_equals_repeated_decode_steps(gdn):
    """The verify kernel runs each token exactly as a decode step does: bit-identical results."""
    N, Tv, Hqk, Hv, d = 7, 6, 2, 4, 128
    flush(f"verify vs decode steps N={N} Tv={Tv}")
    inp = make_verify(N, Tv, Hqk, Hv, d, d, "bf16", seed=5)
    dev = to_dev(inp)
    s_ver = dev["state"].clone()
    o_ver = gdn.decode_verify(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], s_ver, scale=1.1)
    s_dec = dev["state"].clone()
    o_dec = torch.stack([gdn.decode_step(dev["q"][:, t].contiguous(), dev["k"][:, t].contiguous(),
                                         dev["v"][:, t].contiguous(), dev["g"][:, t].contiguous(),
                                         dev["beta"][:, t].contiguous(), s_dec, scale=1.1) for t in range(Tv)], 1)
    torch.cuda.synchronize()
    assert torch.equal(o_ver, o_dec)
    assert torch.equal(s_ver, s_dec)


def test_verify_state_out_none_and_separate(gdn):
    """state_out=None leaves every state untouched; a separate state_out leaves state_in untouched."""
    N, Tv, Hqk, Hv, d = 3, 3, 1, 2, 64
    flush("verify state_out variants")
    inp = make_verify(N, Tv, Hqk, Hv, d, d, "fp32", seed=9)
    dev = to_dev(inp)
    s_in = dev["state"].clone()
    o1 = gdn.decode_verify(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], s_in, state_out=None)
    torch.cuda.synchronize()
    assert torch.equal(s_in, dev["state"])
    s_out = torch.full_like(s_in, float("nan"))
    o2 = gdn.decode_verify(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], s_in, state_out=s_out)
    torch.cuda.synchronize()
    assert torch.equal(s_in, dev["state"])
    assert torch.equal(o1, o2)
    _, ref_states = oracle_verify(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["state"])
    assert_close("separate state_out", f64(s_out), ref_states[:, -1], TOL[torch.float32])


def test_verify_full_workload_whole_tensors(gdn, oracle_pool):
    """256 sequences x 32 value heads, 4 drafted tokens from a live 512 MiB state, updated in place: every
    element of o for every token and of the state after the last token against four oracle decode steps
    per sequence (a verify call is that many consecutive decode steps), whole tensors and every
    (sequence, value head) unit."""
    from oracle.parallel import decode_errors

    w = WORKLOADS["verify_n256_t4"]
    flush(f"verify full {w.name}: drawing inputs")
    inp = make_verify(w.N, w.steps, w.Hqk, w.Hv, w.dk, w.dv, w.dtype, seed=0)
    dev = to_dev(inp)
    state = dev["state"].clone()
    o = gdn.decode_verify(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], state)
    torch.cuda.synchronize()
    o_steps = o.transpose(0, 1).cpu()  # [Tv, N, Hv, dv], the decode driver's layout
    fin = state.cpu()
    steps_inp = {name: inp[name].transpose(0, 1) for name in ("q", "k", "v", "g", "beta")}
    steps_inp["state"] = inp["state"]
    flush("  oracle on the host")
    err, secs = decode_errors(oracle_pool, steps_inp, o_steps, fin)
    s = err.summary()
    tol = TOL[torch.bfloat16]
    flush(f"  {w.name}: rel-L2 o {s['rel_l2_o']:.3e} ({w.steps} tokens) state {s['rel_l2_state']:.3e} over "
          f"{s['units']} units; worst unit o {s['worst_unit_o'][0]} {s['worst_unit_o'][1]:.3e}, state "
          f"{s['worst_unit_state'][0]} {s['worst_unit_state'][1]:.3e} (oracle {secs:.1f} s)")
    assert s["finite"] and s["units"] == w.N * w.Hv
    assert s["rel_l2_o"] <= tol and s["rel_l2_state"] <= tol
    assert s["worst_unit_o"][1] <= tol and s["worst_unit_state"][1] <= tol

"""GPU parity of the segmented prefill (a few long bf16 rows, dk = dv = 128, no cu_seqlens: the rows are cut
into segments that run side by side, then a scan over the segments and a correction of the later segments'
outputs) against the fp64 oracle, through the C ABI."""

import numpy as np
import pytest
import torch

from oracle import recurrent
from parity import TOL, assert_close, f64, flush, rel_l2, to_dev

from linear_attention_token_chunked_amd.inputs import make_prefill

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gdn():
    from linear_attention_token_chunked_amd import gdn as m

    return m


def segmented(gdn, B, T, Hv):
    dims = gdn.make_dims(B, T, B, 1, Hv, 128, 128, 64, 1.0, torch.bfloat16)
    return gdn.fwd_chunked_workspace_size(dims) > 0


@pytest.mark.parametrize("B,T,Hqk,Hv,init,scale", [
    (1, 4096, 1, 2, True, 1.0),    # four segments of 1024 tokens
    (2, 5000, 1, 2, True, 0.09),   # ragged: the last segment ends in a partial chunk
    (1, 8192, 2, 4, False, 1.0),   # grouped heads, zero initial state
])
def test_segmented_matches_oracle(gdn, B, T, Hqk, Hv, init, scale):
    assert segmented(gdn, B, T, Hv), "these shapes take the segmented path"
    flush(f"segmented B={B} T={T} Hqk={Hqk} Hv={Hv} init={init}")
    inp = make_prefill(B, T, Hqk, Hv, 128, 128, "bf16", init_state=init, seed=T + Hv)
    dev = to_dev(inp)
    o, fin = gdn.fwd_chunked(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], initial_state=dev["initial_state"],
                             scale=scale)
    torch.cuda.synchronize()
    ro, rf = recurrent(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], initial_state=inp["initial_state"],
                       scale=scale)
    tol = TOL[torch.bfloat16]
    go, gf = f64(o), f64(fin)
    e_o = assert_close("o", go, ro, tol)
    e_s = assert_close("final_state", gf, rf, tol)
    for b in range(B):
        for h in range(Hv):
            assert rel_l2(go[b, :, h], ro[b, :, h]) <= tol, f"o unit {(b, h)}"
            assert rel_l2(gf[b, h], rf[b, h]) <= tol, f"state unit {(b, h)}"
            # every segment on its own (a wrong start state shows in its tokens first)
            for t0 in range(0, T, 1024):
                assert rel_l2(go[b, t0:t0 + 1024, h], ro[b, t0:t0 + 1024, h]) <= tol, f"o {(b, h)} from {t0}"
    flush(f"  rel-L2 o {e_o:.2e} state {e_s:.2e}")


def test_segmented_slow_decay_carries_state(gdn):
    """Slow gates carry the initial state through every segment: the scan's products must be right."""
    flush("segmented slow decay")
    inp = make_prefill(1, 4096, 1, 2, 128, 128, "bf16", init_state=True, seed=3, gate_scale=0.001)
    dev = to_dev(inp)
    o, fin = gdn.fwd_chunked(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], initial_state=dev["initial_state"])
    torch.cuda.synchronize()
    ro, rf = recurrent(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], initial_state=inp["initial_state"])
    assert_close("o", f64(o), ro, TOL[torch.bfloat16])
    assert_close("final_state", f64(fin), rf, TOL[torch.bfloat16])


def test_segmented_zero_gates(gdn):
    """Full forgets (g = -inf) in the first segment, on a segment boundary and inside the last segment: the
    zero-start and transition runs and the correction stay finite and match the token recurrence."""
    B, T, Hqk, Hv = 1, 4096, 1, 2
    assert segmented(gdn, B, T, Hv), "this shape takes the segmented path"
    flush("segmented zero gates")
    inp = make_prefill(B, T, Hqk, Hv, 128, 128, "bf16", init_state=True, seed=79)
    for t, h in [(500, 0), (1024, 1), (1024, 0), (3000, 1), (4095, 0)]:
        inp["g"][0, t, h] = -float("inf")
    dev = to_dev(inp)
    o, fin = gdn.fwd_chunked(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], initial_state=dev["initial_state"])
    torch.cuda.synchronize()
    ro, rf = recurrent(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], initial_state=inp["initial_state"])
    tol = TOL[torch.bfloat16]
    go, gf = f64(o), f64(fin)
    assert np.all(np.isfinite(go)) and np.all(np.isfinite(gf))
    assert_close("o", go, ro, tol)
    assert_close("final_state", gf, rf, tol)


def test_segmented_equals_unsegmented_path(gdn):
    """The same row through the segmented path and, as one of several rows, through the fused path."""
    flush("segmented vs fused")
    inp = make_prefill(1, 4096, 1, 2, 128, 128, "bf16", init_state=True, seed=4)
    dev = to_dev(inp)
    o1, f1 = gdn.fwd_chunked(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], initial_state=dev["initial_state"])
    # 64 copies of the row make 128 units: too many to segment
    rep = lambda x: x.expand(64, *x.shape[1:]).contiguous()
    o2, f2 = gdn.fwd_chunked(rep(dev["q"]), rep(dev["k"]), rep(dev["v"]), rep(dev["g"]), rep(dev["beta"]),
                             initial_state=rep(dev["initial_state"]))
    torch.cuda.synchronize()
    assert not segmented(gdn, 64, 4096, 2)
    assert rel_l2(f64(o1), f64(o2[:1])) <= 2e-2 and rel_l2(f64(f1), f64(f2[:1])) <= 2e-2


def test_segmented_in_place_state_and_no_final_state(gdn):
    """The final state may overwrite the initial state (the scan writes it after every run has read it), and
    without a final state only the outputs are formed; both match the separate-buffer call bit for bit."""
    flush("segmented in place / no final state")
    inp = make_prefill(1, 4096, 1, 2, 128, 128, "bf16", init_state=True, seed=21)
    dev = to_dev(inp)
    o1, f1 = gdn.fwd_chunked(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], initial_state=dev["initial_state"])
    state = dev["initial_state"].clone()
    o2, f2 = gdn.fwd_chunked(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], initial_state=state,
                             final_state=state)
    o3, f3 = gdn.fwd_chunked(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], initial_state=dev["initial_state"],
                             output_final_state=False)
    torch.cuda.synchronize()
    assert f2 is state and f3 is None
    assert torch.equal(o1, o2) and torch.equal(f1, state) and torch.equal(o1, o3)
    ro, rf = recurrent(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], initial_state=inp["initial_state"])
    assert_close("final_state", f64(state), rf, TOL[torch.bfloat16])

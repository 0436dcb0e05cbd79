"""GPU parity of the two-pass prefill (few (sequence, value head) units in bf16 with dk = dv = 128: a
chunk-parallel pass writes every chunk's T = (I + A)^-1, masked Q K^T and gate vectors to the workspace,
then one workgroup per unit and 32-column slice runs the recurrence from them) against the fp64 oracle,
through the C ABI."""

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


def two_pass(gdn, B, T, N, Hv):
    dims = gdn.make_dims(B, T, N, 1, Hv, 128, 128, 64, 1.0, torch.bfloat16)
    return gdn.fwd_chunked_workspace_size(dims) > 0 and N * Hv <= 128


@pytest.mark.parametrize("B,T,Hqk,Hv,init,scale", [
    (1, 4096, 1, 2, True, 1.0),    # 64 chunks of one row
    (2, 5000, 1, 2, True, 0.09),   # ragged: the last chunk is partial
    (1, 8192, 2, 4, False, 1.0),   # grouped heads, zero initial state
    (4, 700, 4, 32, True, 1.0),    # 128 units: the most the two-pass path takes, four rounds of workgroups
])
def test_two_pass_matches_oracle(gdn, B, T, Hqk, Hv, init, scale):
    assert two_pass(gdn, B, T, B, Hv), "these shapes take the two-pass path"
    flush(f"two-pass B={B} T={T} Hqk={Hqk} Hv={Hv} init={init}")
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
            for t0 in range(0, T, 1024):  # every stretch of the row on its own
                assert rel_l2(go[b, t0:t0 + 1024, h], ro[b, t0:t0 + 1024, h]) <= tol, f"o {(b, h)} from {t0}"
    flush(f"  rel-L2 o {e_o:.2e} state {e_s:.2e}")


def test_two_pass_slow_decay_carries_state(gdn):
    """Slow gates carry the initial state through all 64 chunks: the scan's state update must be right."""
    flush("two-pass slow decay")
    inp = make_prefill(1, 4096, 1, 2, 128, 128, "bf16", init_state=True, seed=3, gate_scale=0.001)
    dev = to_dev(inp)
    o, fin = gdn.fwd_chunked(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], initial_state=dev["initial_state"])
    torch.cuda.synchronize()
    ro, rf = recurrent(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], initial_state=inp["initial_state"])
    assert_close("o", f64(o), ro, TOL[torch.bfloat16])
    assert_close("final_state", f64(fin), rf, TOL[torch.bfloat16])


def test_two_pass_packed_with_empty_and_partial_sequences(gdn):
    """Packed sequences through the two-pass path: chunk offsets formed on the device, empty sequences
    (final = initial, bit for bit), one-token and chunk-boundary lengths, longest first."""
    lens = [0, 1, 63, 64, 65, 700, 0, 129, 2000, 5]
    assert two_pass(gdn, 1, sum(lens), len(lens), 4)
    flush(f"two-pass packed lens={lens}")
    inp = make_prefill(1, 0, 2, 4, 128, 128, "bf16", init_state=True, lengths=lens, seed=31)
    dev = to_dev(inp)
    o, fin = gdn.fwd_chunked(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], initial_state=dev["initial_state"],
                             cu_seqlens=dev["cu_seqlens"])
    torch.cuda.synchronize()
    ro, rf = recurrent(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], initial_state=inp["initial_state"],
                       cu_seqlens=inp["cu_seqlens"])
    tol = TOL[torch.bfloat16]
    go, gf = f64(o), f64(fin)
    assert_close("o", go, ro, tol)
    assert_close("final_state", gf, rf, tol)
    cu = np.concatenate([[0], np.cumsum(lens)])
    for n in range(len(lens)):
        for h in range(4):
            if lens[n]:
                assert rel_l2(go[0, cu[n]:cu[n + 1], h], ro[0, cu[n]:cu[n + 1], h]) <= tol, f"o {(n, h)}"
            assert rel_l2(gf[n, h], rf[n, h]) <= tol, f"state {(n, h)}"
    s0 = f64(inp["initial_state"])
    np.testing.assert_array_equal(gf[0], s0[0])
    np.testing.assert_array_equal(gf[6], s0[6])


def test_two_pass_equals_fused_path(gdn):
    """The same row through the two-pass path and, as one of many rows, through the fused kernel."""
    flush("two-pass vs fused")
    inp = make_prefill(1, 4096, 1, 2, 128, 128, "bf16", init_state=True, seed=4)
    dev = to_dev(inp)
    o1, f1 = gdn.fwd_chunked(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], initial_state=dev["initial_state"])
    # 128 copies of the row make 256 units: the fused kernel
    rep = lambda x: x.expand(128, *x.shape[1:]).contiguous()
    o2, f2 = gdn.fwd_chunked(rep(dev["q"]), rep(dev["k"]), rep(dev["v"]), rep(dev["g"]), rep(dev["beta"]),
                             initial_state=rep(dev["initial_state"]))
    torch.cuda.synchronize()
    assert not two_pass(gdn, 128, 4096, 128, 2)
    assert rel_l2(f64(o1), f64(o2[:1])) <= 2e-2 and rel_l2(f64(f1), f64(f2[:1])) <= 2e-2


def test_two_pass_in_place_state_and_no_final_state(gdn):
    """The final state may overwrite the initial state (each workgroup reads its slice before it writes
    it), and without a final state only the outputs are formed; both match the separate-buffer call bit
    for bit."""
    flush("two-pass in place / no final state")
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

"""GPU parity of gdn_bwd_chunked (gradients of a prefill) against the fp64 autograd oracle, through the C ABI."""

import numpy as np
import pytest
import torch

from oracle import recurrent_grads
from parity import TOL, assert_close, f64, flush, rel_l2, to_dev

from linear_attention_token_chunked_amd.inputs import WORKLOADS, make_cotangents, make_prefill

pytestmark = pytest.mark.gpu
DT = {"bf16": torch.bfloat16, "fp32": torch.float32}
NAMES = ("dq", "dk", "dv", "dg", "dbeta", "d_initial_state")


@pytest.fixture(scope="module")
def gdn():
    from linear_attention_token_chunked_amd import gdn as m

    return m


def run_case(gdn, inp, cot, scale, want_dh0=True):
    dev = to_dev(inp)
    d_o = cot["d_o"].cuda()
    d_fin = cot["d_final"].cuda() if cot["d_final"] is not None else None
    got = gdn.bwd_chunked(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], d_o,
                          initial_state=dev["initial_state"], d_final_state=d_fin, cu_seqlens=dev["cu_seqlens"],
                          scale=scale, want_d_initial_state=want_dh0)
    torch.cuda.synchronize()
    cu = inp["cu_seqlens"].numpy() if inp["cu_seqlens"] is not None else None
    ref = recurrent_grads(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], cot["d_o"], inp["initial_state"],
                          cot["d_final"], cu, scale)
    return got, ref


def check(got, ref, tol, names=NAMES):
    for name in names:
        if got[name] is None:
            continue
        err = assert_close(name, f64(got[name]), ref[name], tol)
        flush(f"  {name}: rel-L2 {err:.2e}")


@pytest.mark.parametrize("dtype,B,T,Hqk,Hv,d,init,final", [
    ("bf16", 2, 200, 2, 4, 128, True, True),     # GQA, three chunks and a ragged tail
    ("bf16", 1, 64, 1, 1, 128, False, False),    # exactly one chunk, no states
    ("bf16", 1, 150, 2, 2, 64, True, False),
    ("fp32", 1, 130, 1, 2, 64, False, True),
    ("fp32", 2, 77, 2, 2, 64, True, True),
])
def test_bwd_small_matches_oracle(gdn, dtype, B, T, Hqk, Hv, d, init, final):
    flush(f"bwd small {dtype} B={B} T={T} Hqk={Hqk} Hv={Hv} d={d} init={init} final={final}")
    inp = make_prefill(B, T, Hqk, Hv, d, d, dtype, init_state=init, seed=T + d)
    cot = make_cotangents(B, T, Hv, d, B, d, dtype, seed=T, final=final)
    got, ref = run_case(gdn, inp, cot, scale=d ** -0.5)
    check(got, ref, TOL[DT[dtype]])


@pytest.mark.parametrize("d,lengths", [
    (128, [0, 70, 1, 129, 64]),
    (64, [5, 0, 300, 63, 65]),
])
def test_bwd_packed_with_empty_sequences(gdn, d, lengths):
    flush(f"bwd packed d={d} lengths={lengths}")
    inp = make_prefill(1, 0, 2, 4, d, d, "bf16", init_state=True, lengths=lengths, seed=3)
    cot = make_cotangents(1, sum(lengths), 4, d, len(lengths), d, "bf16", seed=3)
    got, ref = run_case(gdn, inp, cot, scale=1.0)
    check(got, ref, TOL[torch.bfloat16])
    # an empty sequence passes the final state's gradient straight to the initial state
    for n, L in enumerate(lengths):
        if L == 0:
            assert torch.equal(got["d_initial_state"][n].cpu(), cot["d_final"][n])


@pytest.mark.parametrize("d", [128, 64])
def test_bwd_many_units_wide_launch(gdn, d):
    """64 short packed sequences x 4 value heads = 256 units: the launch shape for wide batches."""
    rng = np.random.default_rng(11)
    lengths = [int(x) for x in rng.integers(1, 40, 64)]
    flush(f"bwd wide d={d} tokens={sum(lengths)}")
    inp = make_prefill(1, 0, 2, 4, d, d, "bf16", init_state=True, lengths=lengths, seed=5)
    cot = make_cotangents(1, sum(lengths), 4, d, 64, d, "bf16", seed=5)
    got, ref = run_case(gdn, inp, cot, scale=d ** -0.5)
    check(got, ref, TOL[torch.bfloat16])


def test_bwd_without_initial_state_gradient(gdn):
    flush("bwd want_d_initial_state=False")
    inp = make_prefill(1, 100, 1, 2, 64, 64, "bf16", init_state=True, seed=8)
    cot = make_cotangents(1, 100, 2, 64, 1, 64, "bf16", seed=8)
    got, ref = run_case(gdn, inp, cot, scale=0.5, want_dh0=False)
    assert got["d_initial_state"] is None
    check(got, ref, TOL[torch.bfloat16], NAMES[:-1])


def test_bwd_repeat_calls_are_identical(gdn):
    """Every gradient is overwritten by each call (nothing accumulates across calls): a second call gives
    the same gradients, up to the order of the in-workgroup sums of dg and dbeta."""
    flush("bwd repeat")
    inp = to_dev(make_prefill(1, 130, 2, 4, 128, 128, "bf16", init_state=True, seed=2))
    cot = make_cotangents(1, 130, 4, 128, 1, 128, "bf16", seed=2)
    args = (inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], cot["d_o"].cuda())
    a = gdn.bwd_chunked(*args, initial_state=inp["initial_state"], d_final_state=cot["d_final"].cuda())
    b = gdn.bwd_chunked(*args, initial_state=inp["initial_state"], d_final_state=cot["d_final"].cuda())
    torch.cuda.synchronize()
    for name in NAMES:
        assert rel_l2(f64(a[name]), f64(b[name])) <= 1e-6, name


def test_bwd_full_workload_sampled_units(gdn):
    """Four sequences of 4096 tokens x 16 heads at d = 128 (one value head per query/key head, so each
    (sequence, head) unit's gradients are the oracle's for that unit alone); oracle on 2 sampled units."""
    w = WORKLOADS["prefill_b4_t4096"]
    flush(f"bwd full {w}")
    inp = make_prefill(w.B, w.T, w.Hqk, w.Hv, w.dk, w.dv, w.dtype, init_state=True, seed=0)
    cot = make_cotangents(w.B, w.T, w.Hv, w.dv, w.B, w.dk, w.dtype, seed=0)
    dev = to_dev(inp)
    got = gdn.bwd_chunked(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], cot["d_o"].cuda(),
                          initial_state=dev["initial_state"], d_final_state=cot["d_final"].cuda(),
                          scale=w.dk ** -0.5)
    torch.cuda.synchronize()
    for name in NAMES:
        assert bool(torch.isfinite(got[name]).all()), name
    for n, h in [(0, 0), (w.B - 1, w.Hv - 1)]:
        flush(f"  unit ({n}, {h})")
        sl = lambda x: x[n:n + 1, :, h:h + 1]
        ref = recurrent_grads(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), sl(inp["g"]), sl(inp["beta"]),
                              sl(cot["d_o"]), inp["initial_state"][n:n + 1, h:h + 1],
                              cot["d_final"][n:n + 1, h:h + 1], None, w.dk ** -0.5)
        for name in NAMES[:-1]:
            assert_close(f"{name} ({n},{h})", f64(got[name][n, :, h]), ref[name][0, :, 0], TOL[torch.bfloat16])
        assert_close(f"d_initial_state ({n},{h})", f64(got["d_initial_state"][n, h]), ref["d_initial_state"][0, 0],
                     TOL[torch.bfloat16])

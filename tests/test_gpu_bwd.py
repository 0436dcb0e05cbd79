"""GPU parity of gdn_bwd_chunked (gradients of a prefill) against the fp64 autograd oracle, through the C ABI."""

import numpy as np
import pytest
import torch

from oracle import recurrent_grads
from parity import TOL, assert_close, f64, flush, to_dev

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


@pytest.mark.parametrize("d,lengths,Hqk", [
    (128, [0, 70, 1, 129, 64], 2),
    (64, [5, 0, 300, 63, 65], 2),
    (128, [200, 0, 33], 1),  # four value heads on one query/key head
])
def test_bwd_packed_with_empty_sequences(gdn, d, lengths, Hqk):
    flush(f"bwd packed d={d} lengths={lengths} Hqk={Hqk}")
    inp = make_prefill(1, 0, Hqk, 4, d, d, "bf16", init_state=True, lengths=lengths, seed=3)
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


def test_bwd_zero_gates(gdn):
    """Gradients through full forgets (g = -inf): finite everywhere, and matching the autograd oracle, whose
    gradient with respect to such a g is exactly zero (the kernels' is zero up to rounding)."""
    flush("bwd zero gates")
    B, T, Hqk, Hv, d = 2, 200, 2, 4, 128
    inp = make_prefill(B, T, Hqk, Hv, d, d, "bf16", init_state=True, seed=81)
    for b, t, h in [(0, 0, 0), (0, 37, 1), (0, 64, 2), (1, 150, 3), (1, 160, 3), (1, 199, 0)]:
        inp["g"][b, t, h] = -float("inf")
    cot = make_cotangents(B, T, Hv, d, B, d, "bf16", seed=82)
    got, ref = run_case(gdn, inp, cot, scale=d ** -0.5)
    for name in NAMES:
        if got[name] is not None:
            assert np.all(np.isfinite(f64(got[name]))), name
    check(got, ref, TOL[torch.bfloat16])


def test_bwd_rows_without_tokens(gdn):
    """B rows of zero tokens: the final state is the initial state, so its gradient passes through unchanged,
    bit for bit."""
    flush("bwd rows without tokens")
    inp = make_prefill(2, 0, 1, 2, 128, 128, "bf16", init_state=True, seed=16)
    cot = make_cotangents(2, 0, 2, 128, 2, 128, "bf16", seed=17)
    got, _ = run_case(gdn, inp, cot, scale=1.0)
    assert torch.equal(got["d_initial_state"].cpu(), cot["d_final"])
    assert got["dq"].numel() == 0 and got["dv"].numel() == 0


def test_bwd_without_initial_state_gradient(gdn):
    flush("bwd want_d_initial_state=False")
    inp = make_prefill(1, 100, 1, 2, 64, 64, "bf16", init_state=True, seed=8)
    cot = make_cotangents(1, 100, 2, 64, 1, 64, "bf16", seed=8)
    got, ref = run_case(gdn, inp, cot, scale=0.5, want_dh0=False)
    assert got["d_initial_state"] is None
    check(got, ref, TOL[torch.bfloat16], NAMES[:-1])


def test_bwd_repeat_calls_are_identical(gdn):
    """Every gradient is overwritten by each call (nothing accumulates across calls), and every sum is taken
    in a fixed order (no atomics): repeated calls give bitwise the same gradients, also when value heads
    share a query/key head and sequences are packed."""
    flush("bwd repeat")
    for lengths, Hqk, Hv in [(None, 2, 4), ([130, 7, 300, 64], 1, 4)]:
        T = 130 if lengths is None else 0
        inp = to_dev(make_prefill(1, T, Hqk, Hv, 128, 128, "bf16", init_state=True, lengths=lengths, seed=2))
        N = 1 if lengths is None else len(lengths)
        tokens = inp["q"].shape[1]
        cot = make_cotangents(1, tokens, Hv, 128, N, 128, "bf16", seed=2)
        args = (inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], cot["d_o"].cuda())
        kw = dict(initial_state=inp["initial_state"], d_final_state=cot["d_final"].cuda(),
                  cu_seqlens=inp["cu_seqlens"], scale=128 ** -0.5)
        a = gdn.bwd_chunked(*args, **kw)
        for _ in range(2):
            b = gdn.bwd_chunked(*args, **kw)
            torch.cuda.synchronize()
            for name in NAMES:
                assert torch.equal(a[name], b[name]), (lengths, name)


def test_bwd_full_workload_whole_tensors(gdn, oracle_grad_pool):
    """Four sequences of 4096 tokens x 16 heads at d = 128: every element of every gradient against the
    fp64 autograd oracle (one piece per (sequence, head), on forked host processes), as whole tensors and
    per unit."""
    from oracle.parallel import GRADS, bwd_errors

    w = WORKLOADS["prefill_b4_t4096"]
    flush(f"bwd full {w.name}: drawing inputs")
    inp = make_prefill(w.B, w.T, w.Hqk, w.Hv, w.dk, w.dv, w.dtype, init_state=True, seed=0)
    cot = make_cotangents(w.B, w.T, w.Hv, w.dv, w.B, w.dk, w.dtype, seed=0)
    dev = to_dev(inp)
    got = gdn.bwd_chunked(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], cot["d_o"].cuda(),
                          initial_state=dev["initial_state"], d_final_state=cot["d_final"].cuda(),
                          scale=w.dk ** -0.5)
    torch.cuda.synchronize()
    got = {key: got[key].cpu() for key in GRADS}
    flush("  oracle on the host (about 40 s per piece, 64 pieces)")
    err, secs = bwd_errors(oracle_grad_pool, inp, cot, got, scale=w.dk ** -0.5,
                           progress=lambda done, total: flush(f"  piece {done}/{total}"))
    tol = TOL[torch.bfloat16]
    assert err.finite
    for key in GRADS:
        unit, worst = err.worst(key)
        flush(f"  {key}: rel-L2 {err.rel(key):.3e}, worst unit {unit} {worst:.3e}")
        assert err.rel(key) <= tol and worst <= tol, key
    flush(f"  oracle {secs:.0f} s")

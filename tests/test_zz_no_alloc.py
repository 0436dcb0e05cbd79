"""gdn_fwd_chunked_noalloc (through the C ABI) against gdn_fwd_chunked, two calls in a row, the second
with a smaller input: the static scratch keeps the first call's contents and must not leak into the
second.  Packed sequences take the same kernels and the same order on both entry points, so the
results agree bit for bit; a long row that gdn_fwd_chunked cuts into segments runs in one pass of the
fused kernel here and agrees within the bf16 parity bar."""

import numpy as np
import pytest
import torch

from parity import TOL, assert_close, f64, flush, rel_l2, to_dev

from linear_attention_token_chunked_amd.inputs import make_prefill, packed_lengths

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gdn():
    from linear_attention_token_chunked_amd import gdn as m

    return m


def both(gdn, inp):
    d = to_dev(inp)
    B, T, _, dk = d["q"].shape
    Hv = d["v"].shape[2]
    N = B if d["cu_seqlens"] is None else d["cu_seqlens"].shape[0] - 1
    o_ws, f_ws = gdn.fwd_chunked(d["q"], d["k"], d["v"], d["g"], d["beta"], initial_state=d["initial_state"],
                                 cu_seqlens=d["cu_seqlens"])
    o_na = torch.full_like(o_ws, float("nan"))
    f_na = torch.full((N, Hv, dk, dk), float("nan"), device=o_ws.device)
    gdn.fwd_chunked_noalloc(d["q"], d["k"], d["v"], d["g"], d["beta"], initial_state=d["initial_state"],
                            cu_seqlens=d["cu_seqlens"], out=o_na, final_state=f_na)
    torch.cuda.synchronize()
    return o_ws, f_ws, o_na, f_na


def test_no_alloc_packed_two_calls_second_smaller(gdn):
    rng = np.random.default_rng(41)
    for n, Hqk, Hv in ((96, 2, 4), (9, 1, 2)):  # 96 sequences (ordered in the scratch), then 9
        lens = [int(x) for x in np.minimum(packed_lengths(rng, n), 700)]
        lens[1] = 0
        flush(f"no-alloc packed N={n} tokens={sum(lens)} Hqk={Hqk} Hv={Hv}")
        inp = make_prefill(1, 0, Hqk, Hv, 128, 128, "bf16", init_state=True, lengths=lens, seed=n)
        o_ws, f_ws, o_na, f_na = both(gdn, inp)
        assert torch.equal(o_ws, o_na) and torch.equal(f_ws, f_na)


def test_no_alloc_long_row_runs_fused(gdn):
    """A long row with two heads: segments through gdn_fwd_chunked, one fused pass without allocation."""
    flush("no-alloc long row")
    inp = make_prefill(1, 4096, 1, 2, 128, 128, "bf16", init_state=True, seed=42)
    o_ws, f_ws, o_na, f_na = both(gdn, inp)
    assert bool(torch.isfinite(o_na.float()).all()) and bool(torch.isfinite(f_na).all())
    tol = TOL[torch.bfloat16]
    assert rel_l2(f64(o_na), f64(o_ws)) <= tol and rel_l2(f64(f_na), f64(f_ws)) <= tol
    from oracle import recurrent

    ro, rf = recurrent(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], initial_state=inp["initial_state"])
    assert_close("o", f64(o_na), ro, tol)
    assert_close("final_state", f64(f_na), rf, tol)

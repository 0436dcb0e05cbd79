"""GPU parity of gdn_fwd_chunked against the fp64 oracle (through the C ABI).

Every case compares every element of o and of the final states with the
oracle's token recurrence.  Small cases span several chunks and a ragged tail;
the full-size workloads run in the launch configuration the bench times, with
the oracle spread over forked host processes.
"""

import numpy as np
import pytest
import torch

from oracle import recurrent
from parity import TOL, assert_close, f64, flush, rel_l2, to_dev, whole_check

from linear_attention_token_chunked_amd.inputs import WORKLOADS, make_prefill

pytestmark = pytest.mark.gpu
DT = {"bf16": torch.bfloat16, "fp32": torch.float32}


@pytest.fixture(scope="module")
def gdn():
    from linear_attention_token_chunked_amd import gdn as m

    return m


def run_gpu(gdn, inp, **kw):
    dev = to_dev(inp)
    o, fin = gdn.fwd_chunked(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"],
                             initial_state=dev.get("initial_state"), cu_seqlens=dev.get("cu_seqlens"), **kw)
    torch.cuda.synchronize()
    return o, fin


def check_against_oracle(gdn, inp, dtype, scale=1.0, per_unit=True):
    o, fin = run_gpu(gdn, inp, scale=scale)
    ro, rf = recurrent(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], initial_state=inp.get("initial_state"),
                       cu_seqlens=inp.get("cu_seqlens"), scale=scale)
    tol = TOL[DT[dtype]]
    go, gf = f64(o), f64(fin)
    e_o = assert_close("o", go, ro, tol)
    e_s = assert_close("final_state", gf, rf, tol)
    if per_unit:  # a single broken head must not hide inside the global norm
        Hv = go.shape[2]
        for h in range(Hv):
            if np.linalg.norm(ro[:, :, h]) > 0:
                assert rel_l2(go[:, :, h], ro[:, :, h]) <= tol, f"o head {h}"
        for n in range(gf.shape[0]):
            for h in range(Hv):
                if np.linalg.norm(rf[n, h]) > 0:
                    assert rel_l2(gf[n, h], rf[n, h]) <= tol, f"state {(n, h)}"
    flush(f"  rel-L2 o {e_o:.2e} state {e_s:.2e}")
    return go, gf


def test_tiny_fp32_workload(gdn):
    """B=1, T=256, H=2, dk=dv=64, fp32, zero initial state, seed 0: tolerance 1e-5."""
    w = WORKLOADS["tiny_fp32"]
    flush(f"prefill {w.name}")
    inp = make_prefill(w.B, w.T, w.Hqk, w.Hv, w.dk, w.dv, w.dtype, init_state=False, seed=0)
    check_against_oracle(gdn, inp, "fp32")


@pytest.mark.parametrize("dtype,B,T,Hqk,Hv,d,init", [
    ("bf16", 2, 300, 2, 4, 128, True),    # several chunks + a ragged tail, grouped heads
    ("bf16", 1, 200, 1, 1, 128, False),
    ("bf16", 2, 130, 2, 2, 64, True),
    ("fp32", 2, 257, 1, 2, 64, True),
    ("fp32", 1, 1, 1, 1, 64, True),       # one token
    ("bf16", 1, 64, 4, 8, 128, True),     # exactly one chunk
])
def test_small_shapes(gdn, dtype, B, T, Hqk, Hv, d, init):
    flush(f"prefill small {dtype} B={B} T={T} Hqk={Hqk} Hv={Hv} d={d} init={init}")
    inp = make_prefill(B, T, Hqk, Hv, d, d, dtype, init_state=init, seed=B * 1000 + T)
    check_against_oracle(gdn, inp, dtype, scale=0.9)


@pytest.mark.parametrize("B,T,Hqk,Hv,d", [
    (3, 150, 8, 16, 128),    # 48 (sequence, head) units: 32-wide slices
    (8, 130, 8, 16, 128),    # 128 units: 64-wide
    (16, 70, 8, 16, 128),    # 256 units: whole rows
    (8, 100, 4, 16, 64),     # 128 units, dk = dv = 64: whole rows
])
def test_unit_counts_of_every_slice_width(gdn, B, T, Hqk, Hv, d):
    """The kernel splits the state columns into 32, 64 or 128-wide slices depending on how many
    (sequence, head) units there are; the small shapes above take the narrowest, these the
    others (and a ragged last chunk in each)."""
    flush(f"prefill units={B * Hv} B={B} T={T} Hqk={Hqk} Hv={Hv} d={d}")
    inp = make_prefill(B, T, Hqk, Hv, d, d, "bf16", init_state=True, seed=B * 100 + T)
    check_against_oracle(gdn, inp, "bf16", scale=1.1)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("fp32", 64)])
def test_packed_ragged_lengths(gdn, dtype, d):
    """Packed batch with empty, 1-token, chunk-boundary and ragged sequences."""
    lens = [0, 1, 15, 16, 63, 64, 65, 129, 0, 200]
    flush(f"prefill packed {dtype} d={d} lens={lens}")
    inp = make_prefill(1, 0, 2, 4, d, d, dtype, init_state=True, lengths=lens, seed=5)
    go, gf = check_against_oracle(gdn, inp, dtype)
    s0 = f64(inp["initial_state"])
    np.testing.assert_array_equal(gf[0], s0[0])  # empty sequence: final == initial, bit for bit
    np.testing.assert_array_equal(gf[8], s0[8])


def test_many_packed_sequences_longest_first(gdn):
    """300 packed sequences of random lengths with many ties: their workgroups run longest first
    (an order formed on the device over more than one block of sequences); results are per sequence."""
    rng = np.random.default_rng(11)
    lens = [int(x) for x in rng.integers(0, 131, size=300)]
    lens[7] = 700  # one long sequence among short ones
    flush(f"prefill packed N={len(lens)} tokens={sum(lens)}")
    inp = make_prefill(1, 0, 1, 2, 64, 64, "bf16", init_state=True, lengths=lens, seed=12)
    check_against_oracle(gdn, inp, "bf16")


def test_packed_beyond_ordering_limit(gdn):
    """More than 4096 packed sequences keep their natural order (no ordering workspace): still per sequence."""
    rng = np.random.default_rng(13)
    lens = [int(x) for x in rng.integers(0, 9, size=4200)]
    lens[100] = 300
    flush(f"prefill packed N={len(lens)} tokens={sum(lens)} (natural order)")
    inp = make_prefill(1, 0, 1, 1, 64, 64, "bf16", init_state=True, lengths=lens, seed=14)
    dims = gdn.make_dims(1, sum(lens), len(lens), 1, 1, 64, 64, 64, 1.0, torch.bfloat16)
    assert gdn.fwd_chunked_workspace_size(dims) == 0
    check_against_oracle(gdn, inp, "bf16")


def test_slow_decay_long_carry(gdn):
    """log(alpha) scaled by 0.001: the state carries across all chunks and the initial state stays visible."""
    flush("prefill slow decay")
    inp = make_prefill(1, 1024, 1, 2, 128, 128, "bf16", init_state=True, seed=9, gate_scale=0.001)
    check_against_oracle(gdn, inp, "bf16")


def test_identity_gates_keep_state_and_read_it(gdn):
    """alpha = 1, beta = 0: final == initial and o_t = M0^T q_t (fp32, tolerance 1e-5)."""
    inp = make_prefill(1, 150, 1, 2, 64, 64, "fp32", init_state=True, seed=3)
    inp["g"].zero_()
    inp["beta"].zero_()
    o, fin = run_gpu(gdn, inp)
    s0 = f64(inp["initial_state"])
    assert_close("final", f64(fin), s0, 1e-6)
    expect = np.einsum("ti,hij->thj", f64(inp["q"])[0, :, 0], s0[0])
    assert_close("o", f64(o)[0], expect, 1e-5)


def test_query_equal_key_beta_one_reads_back_value(gdn):
    """beta = 1, unit keys, q = k: o_t = v_t for any history (fp32)."""
    inp = make_prefill(1, 200, 1, 1, 64, 64, "fp32", init_state=True, seed=4)
    inp["beta"].fill_(1.0)
    inp["q"] = inp["k"].clone()
    o, _ = run_gpu(gdn, inp)
    assert_close("o", f64(o), f64(inp["v"]), 1e-5)


# (batch row, token, value head) of the full-forget gates: a sequence's first token, inside a chunk, both sides
# of a chunk boundary, twice in one chunk, the last token
ZERO_GATES = [(0, 0, 0), (0, 37, 1), (0, 63, 2), (0, 64, 2), (1, 150, 3), (1, 160, 3), (1, 299, 0), (1, 100, 1)]


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("fp32", 64)])
def test_zero_gates_erase_history(gdn, dtype, d):
    """alpha = 0 (g = -inf, the full forget) on tokens of every kind of place, and one finite gate far below
    the kernels' floor: o and the final states stay finite and match the token recurrence."""
    flush(f"prefill zero gates {dtype} d={d}")
    inp = make_prefill(2, 300, 2, 4, d, d, dtype, init_state=True, seed=77 + d)
    for b, t, h in ZERO_GATES:
        inp["g"][b, t, h] = -float("inf")
    inp["g"][0, 200, 3] = -1e4
    go, gf = check_against_oracle(gdn, inp, dtype, scale=0.9)
    assert np.all(np.isfinite(go)) and np.all(np.isfinite(gf))


def test_zero_gates_packed(gdn):
    """The same in a packed batch: a full forget on a sequence's first token, at a chunk boundary and last."""
    lens = [70, 0, 130, 64]
    flush(f"prefill zero gates packed lens={lens}")
    inp = make_prefill(1, 0, 2, 4, 128, 128, "bf16", init_state=True, lengths=lens, seed=78)
    for t, h in [(0, 0), (70, 1), (70 + 64, 2), (199, 3), (200, 0), (263, 1)]:
        inp["g"][0, t, h] = -float("inf")
    go, gf = check_against_oracle(gdn, inp, "bf16")
    assert np.all(np.isfinite(go)) and np.all(np.isfinite(gf))


@pytest.mark.parametrize("dtype,d,init", [("bf16", 128, True), ("bf16", 128, False), ("fp32", 64, True)])
def test_rows_without_tokens(gdn, dtype, d, init):
    """B rows of zero tokens: nothing to run, and every final state is the initial one, bit for bit (zeros
    without an initial state)."""
    flush(f"prefill rows without tokens {dtype} d={d} init={init}")
    inp = make_prefill(2, 0, 1, 2, d, d, dtype, init_state=init, seed=15)
    o, fin = run_gpu(gdn, inp)
    assert o.shape == (2, 0, 2, d)
    expect = inp["initial_state"] if init else torch.zeros((2, 2, d, d))
    assert torch.equal(fin.cpu(), expect)


def test_max_value_heads(gdn):
    """The largest head count the boundary accepts, 4096 value heads over 2048 q/k heads, d = 128: a token row
    of v and o is 1 MB, the largest stride the kernels' 32-bit row offsets take.  Two chunks with a ragged tail;
    every output is finite, and the first and last heads (the largest offsets) match the oracle element by
    element (the oracle runs on those heads alone: the heads are independent recurrences)."""
    Hqk, Hv, T = 2048, 4096, 70
    flush(f"prefill max heads Hqk={Hqk} Hv={Hv} T={T}")
    inp = make_prefill(1, T, Hqk, Hv, 128, 128, "bf16", init_state=True, seed=19)
    o, fin = run_gpu(gdn, inp, scale=0.9)
    go, gf = f64(o), f64(fin)
    assert np.all(np.isfinite(go)) and np.all(np.isfinite(gf))
    heads = [0, 1, 2047, 2048, 4094, 4095]
    qk = [h // (Hv // Hqk) for h in heads]
    ro, rf = recurrent(inp["q"][:, :, qk], inp["k"][:, :, qk], inp["v"][:, :, heads], inp["g"][:, :, heads],
                       inp["beta"][:, :, heads], initial_state=inp["initial_state"][:, heads], scale=0.9)
    tol = TOL[torch.bfloat16]
    for i, h in enumerate(heads):
        assert rel_l2(go[:, :, h], ro[:, :, i]) <= tol, f"o head {h}"
        assert rel_l2(gf[:, h], rf[:, i]) <= tol, f"state head {h}"


def test_in_place_state_and_no_final_state(gdn):
    inp = make_prefill(2, 100, 1, 2, 128, 128, "bf16", init_state=True, seed=6)
    dev = to_dev(inp)
    o_ref, f_ref = gdn.fwd_chunked(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"],
                                   initial_state=dev["initial_state"])
    st = dev["initial_state"].clone()
    o_inp, f_inp = gdn.fwd_chunked(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], initial_state=st,
                                   final_state=st)
    o_nf, f_nf = gdn.fwd_chunked(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"],
                                 initial_state=dev["initial_state"], output_final_state=False)
    torch.cuda.synchronize()
    assert f_nf is None
    assert torch.equal(o_ref, o_inp) and torch.equal(o_ref, o_nf)
    assert torch.equal(f_ref, st)


def test_composition_and_decode_continuity(gdn):
    """prefill(T1) then prefill(T2, init = final) == prefill(T1 + T2); decode steps == prefill."""
    inp = make_prefill(1, 160, 2, 2, 128, 128, "bf16", init_state=True, seed=8)
    dev = to_dev(inp)
    o_all, f_all = gdn.fwd_chunked(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"],
                                   initial_state=dev["initial_state"])
    sl = lambda x, a, b: x[:, a:b].contiguous()
    o_a, f_a = gdn.fwd_chunked(*(sl(dev[x], 0, 70) for x in ("q", "k", "v", "g", "beta")),
                               initial_state=dev["initial_state"])
    o_b, f_b = gdn.fwd_chunked(*(sl(dev[x], 70, 160) for x in ("q", "k", "v", "g", "beta")), initial_state=f_a)
    assert rel_l2(f64(torch.cat([o_a, o_b], 1)), f64(o_all)) < 5e-3
    assert rel_l2(f64(f_b), f64(f_all)) < 5e-3
    state = dev["initial_state"].clone()
    outs = [gdn.decode_step(dev["q"][:, t].contiguous(), dev["k"][:, t].contiguous(), dev["v"][:, t].contiguous(),
                            dev["g"][:, t].contiguous(), dev["beta"][:, t].contiguous(), state) for t in range(160)]
    assert rel_l2(f64(torch.stack(outs, 1)), f64(o_all)) < 2e-2
    assert rel_l2(f64(state), f64(f_all)) < 2e-2


def test_one_packed_sequence_equals_the_row(gdn):
    """cu_seqlens = {0, T} is the single batch row: same path, bit-identical results."""
    inp = make_prefill(1, 4096, 1, 2, 128, 128, "bf16", init_state=True, seed=21)
    o1, f1 = run_gpu(gdn, inp)
    packed = dict(inp, cu_seqlens=torch.tensor([0, 4096], dtype=torch.int32))
    o2, f2 = run_gpu(gdn, packed)
    assert torch.equal(o1, o2) and torch.equal(f1, f2)


@pytest.mark.parametrize("case", ["batch", "packed", "segmented"])
def test_deterministic(gdn, case):
    """Repeated calls are bit-identical: no atomics, and the orders (longest-first sequences, the
    segments' scan) are fixed by the inputs."""
    if case == "batch":
        inp = make_prefill(2, 300, 2, 4, 128, 128, "bf16", init_state=True, seed=12)
    elif case == "packed":
        inp = make_prefill(1, 0, 2, 4, 128, 128, "bf16", init_state=True, lengths=[300, 7, 300, 0, 129, 64], seed=12)
    else:
        inp = make_prefill(1, 4096, 1, 2, 128, 128, "bf16", init_state=True, seed=12)
    o1, f1 = run_gpu(gdn, inp)
    o2, f2 = run_gpu(gdn, inp)
    assert torch.equal(o1, o2) and torch.equal(f1, f2)


# ----------------------------------------------------------------------------- full sizes
def whole_workload_check(gdn, pool, name):
    """Every element of o and of every final state, at the workload's full size and in the launch
    configuration the bench times, against the oracle's token recurrence (run on forked host
    processes, one piece per (sequence, query/key head)); the bar holds for the whole tensors and
    for every (sequence, value head) unit on its own."""
    w = WORKLOADS[name]
    flush(f"prefill full {w.name}: drawing inputs")
    inp = make_prefill(w.B, w.T, w.Hqk, w.Hv, w.dk, w.dv, w.dtype, init_state=w.init_state, seed=0,
                       num_packed=w.num_packed)
    flush(f"  tokens {inp['q'].shape[0] * inp['q'].shape[1]}: GPU")
    o, fin = run_gpu(gdn, inp)
    o, fin = o.cpu(), fin.cpu()
    flush("  oracle on the host")
    s = whole_check(pool, inp, o, fin, TOL[DT[w.dtype]], w.name)
    return s


def test_full_prefill_b4_t4096(gdn, oracle_pool):
    s = whole_workload_check(gdn, oracle_pool, "prefill_b4_t4096")
    assert s["units"] == 64


def test_full_prefill_t65536_gqa(gdn, oracle_pool):
    s = whole_workload_check(gdn, oracle_pool, "prefill_t65536_gqa")
    assert s["units"] == 32


def test_full_varlen_64(gdn, oracle_pool):
    s = whole_workload_check(gdn, oracle_pool, "varlen_64")
    assert s["units"] == 64 * 32

"""The parallel oracle driver (oracle/parallel.py) that the full-size GPU parity tests use.

It must return the oracle's own result as error-free, find a planted error in the
one unit that holds it, transport bf16 values exactly, reproduce the serial
oracle's decode steps, and cut the backward into pieces whose gradients equal the
whole-input autograd oracle's (dq and dk summed over grouped value heads).  CPU only.
"""

import numpy as np
import torch

from oracle import decode_step, recurrent, recurrent_grads
from oracle.parallel import GRADS, _pack, _unpack, bwd_errors, decode_errors, prefill_errors

from linear_attention_token_chunked_amd.inputs import make_cotangents, make_decode, make_prefill


def _as_candidate(x, dtype):
    return torch.from_numpy(np.asarray(x, np.float32)).to(dtype)


def test_bf16_transport_is_exact():
    x = torch.randn(1000).to(torch.bfloat16)
    x[:4] = torch.tensor([0.0, -0.0, float("inf"), -3.5])
    back = _unpack(_pack(x))
    np.testing.assert_array_equal(back, x.to(torch.float64).numpy())
    y = torch.randn(33)
    np.testing.assert_array_equal(_unpack(_pack(y)), y.to(torch.float64).numpy())


def test_prefill_oracle_result_has_rounding_error_only(oracle_pool):
    inp = make_prefill(2, 70, 2, 4, 16, 8, "fp32", init_state=True, seed=3)
    ro, rf = recurrent(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], initial_state=inp["initial_state"])
    err, _, tokens = prefill_errors(oracle_pool, inp, _as_candidate(ro, torch.float32),
                                    _as_candidate(rf, torch.float32))
    s = err.summary()
    assert tokens == 140 and s["units"] == 8 and s["finite"]
    assert s["rel_l2_o"] < 1e-6 and s["rel_l2_state"] < 1e-6


def test_prefill_planted_error_lands_in_its_unit(oracle_pool):
    lens = [5, 0, 90, 33]
    inp = make_prefill(1, 0, 1, 2, 16, 16, "bf16", init_state=True, lengths=lens, seed=4)
    ro, rf = recurrent(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], initial_state=inp["initial_state"],
                       cu_seqlens=inp["cu_seqlens"])
    o = _as_candidate(ro, torch.bfloat16)
    fin = _as_candidate(rf, torch.float32)
    o[0, 5 + 7, 1] *= -1.0  # sequence 2 covers tokens 5..94: a wrong sign in one token of (2, 1)
    fin[3, 0, 2, 2] += 1.0
    err, _, _ = prefill_errors(oracle_pool, inp, o, fin)
    assert err.worst("o")[0] == (2, 1) and err.worst("o")[1] > 0.05
    assert err.unit["o"][(2, 0)] < 1e-2 and err.unit["o"][(3, 1)] < 1e-2
    assert err.worst("state")[0] == (3, 0)
    # the empty sequence: final == initial, compared as a state unit
    assert err.unit["state"][(1, 0)] < 1e-7


def test_decode_driver_equals_serial_steps(oracle_pool):
    inp = make_decode(3, 2, 4, 16, 8, steps=5, dtype="bf16", seed=2)
    s = inp["state"].double().numpy()
    outs = []
    for t in range(5):
        o, s = decode_step(inp["q"][t], inp["k"][t], inp["v"][t], inp["g"][t], inp["beta"][t], s)
        outs.append(o)
    o_all = np.stack(outs)
    err, _ = decode_errors(oracle_pool, inp, _as_candidate(o_all, torch.float32), _as_candidate(s, torch.float32))
    assert err.units == 12 and err.rel("o") < 1e-6 and err.rel("state") < 1e-6
    bad = _as_candidate(o_all, torch.float32)
    bad[4, 2, 3] = 0.0  # the last step of unit (2, 3)
    err, _ = decode_errors(oracle_pool, inp, bad, _as_candidate(s, torch.float32))
    assert err.worst("o")[0] == (2, 3)


def test_bwd_driver_equals_whole_input_autograd(oracle_grad_pool):
    """Packed sequences (one empty) with two value heads per query/key head: the pieces' gradients
    equal those of one autograd pass over the whole input, and a planted error lands in its unit."""
    lens = [9, 0, 40, 17]
    inp = make_prefill(1, 0, 2, 4, 8, 8, "fp32", init_state=True, lengths=lens, seed=6)
    cot = make_cotangents(1, sum(lens), 4, 8, len(lens), 8, "fp32", seed=6)
    ref = recurrent_grads(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], cot["d_o"], inp["initial_state"],
                          cot["d_final"], inp["cu_seqlens"].numpy(), 0.7)
    cand = {key: _as_candidate(ref[key], torch.float32) for key in GRADS}
    err, _ = bwd_errors(oracle_grad_pool, inp, cot, cand, scale=0.7)
    assert err.finite and err.units == 4 * 2  # (sequence, query/key head) pieces
    for key in GRADS:
        assert err.rel(key) < 1e-6, key
    assert len(err.unit["dv"]) == 4 * 4 and len(err.unit["dq"]) == 4 * 2
    bad = dict(cand)
    bad["dg"] = cand["dg"].clone()
    bad["dg"][0, 9 + 30, 3] += 5.0  # sequence 2 covers tokens 9..48: unit (2, 3)
    err, _ = bwd_errors(oracle_grad_pool, inp, cot, bad, scale=0.7)
    assert err.worst("dg")[0] == (2, 3) and err.unit["dg"][(2, 2)] < 1e-6
    assert err.rel("dq") < 1e-6

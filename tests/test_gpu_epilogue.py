"""GPU parity of gdn_output_norm_gate (zero-centred RMSNorm + sigmoid output gate) against the
fp64 oracle, through the C ABI."""

import numpy as np
import pytest
import torch

from oracle import output_norm_gate as oracle_norm_gate
from parity import TOL, assert_close, f64, flush, to_dev

from linear_attention_token_chunked_amd.inputs import make_epilogue

pytestmark = pytest.mark.gpu
DT = {"bf16": torch.bfloat16, "fp32": torch.float32}


@pytest.fixture(scope="module")
def gdn():
    from linear_attention_token_chunked_amd import gdn as m

    return m


@pytest.mark.parametrize("dtype,rows,dv,eps", [
    ("bf16", 1000, 128, 1e-6),
    ("fp32", 777, 128, 1e-6),
    ("bf16", 513, 64, 1e-5),
    ("fp32", 3, 64, 0.0),
    ("bf16", 1, 128, 1e-6),
])
def test_norm_gate_matches_oracle(gdn, dtype, rows, dv, eps):
    flush(f"norm gate {dtype} rows={rows} dv={dv} eps={eps}")
    inp = make_epilogue(rows, dv, dtype, seed=rows)
    dev = to_dev(inp)
    y = gdn.output_norm_gate(dev["o"], dev["z"], dev["w"], eps=eps)
    ref = oracle_norm_gate(inp["o"], inp["z"], inp["w"], eps=eps)
    tol = TOL[DT[dtype]]
    assert_close("y", f64(y), ref, tol)
    # every row on its own too
    err = np.linalg.norm(f64(y) - ref, axis=-1) / np.linalg.norm(ref, axis=-1)
    assert float(err.max()) <= (2e-2 if dtype == "bf16" else 1e-5), float(err.max())


def test_norm_gate_in_place_and_shapes(gdn):
    """y may be o itself; any leading shape is rows (a prefill output [B, T, Hv, dv])."""
    flush("norm gate in place [2, 37, 4, 128]")
    inp = make_epilogue(2 * 37 * 4, 128, "bf16", seed=3)
    o = inp["o"].reshape(2, 37, 4, 128)
    z = inp["z"].reshape(2, 37, 4, 128)
    dev_o, dev_z, dev_w = o.cuda(), z.cuda(), inp["w"].cuda()
    y_sep = gdn.output_norm_gate(dev_o, dev_z, dev_w)
    gdn.output_norm_gate(dev_o, dev_z, dev_w, out=dev_o)
    torch.cuda.synchronize()
    assert torch.equal(dev_o, y_sep)
    assert_close("y", f64(dev_o), oracle_norm_gate(o, z, inp["w"]), TOL[torch.bfloat16])


def test_norm_gate_full_prefill_output(gdn):
    """The output of prefill_b4_t4096 (4 x 4096 tokens x 16 heads x 128 = 262144 rows): every element against
    the oracle, as a whole tensor and row by row."""
    rows, dv = 4 * 4096 * 16, 128
    flush(f"norm gate full rows={rows}")
    inp = make_epilogue(rows, dv, "bf16", seed=0)
    dev = to_dev(inp)
    y = gdn.output_norm_gate(dev["o"], dev["z"], dev["w"])
    torch.cuda.synchronize()
    got = f64(y)
    ref = oracle_norm_gate(inp["o"], inp["z"], inp["w"])
    tol = TOL[torch.bfloat16]
    err = assert_close("y", got, ref, tol)
    per_row = np.sqrt(((got - ref) ** 2).sum(-1) / np.maximum((ref ** 2).sum(-1), 1e-300))
    flush(f"  rel-L2 {err:.2e}, worst row {per_row.max():.2e}")
    assert per_row.max() <= tol

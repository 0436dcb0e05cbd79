"""GPU parity of gdn_short_conv (short causal convolution along the tokens, per channel, with
optional per-head L2 normalisation) against the fp64 oracle, through the C ABI."""

import numpy as np
import pytest
import torch

from oracle import short_conv as oracle_conv
from parity import TOL, assert_close, f64, flush

from linear_attention_token_chunked_amd.inputs import make_conv

pytestmark = pytest.mark.gpu
DT = {"bf16": torch.bfloat16, "fp32": torch.float32}


@pytest.fixture(scope="module")
def gdn():
    from linear_attention_token_chunked_amd import gdn as m

    return m


@pytest.mark.parametrize("dtype,B,T,H,hd,l2,packed", [
    ("bf16", 2, 70, 4, 128, True, 0),
    ("bf16", 1, 300, 2, 128, False, 5),    # packed, several sequences, some shorter than the taps
    ("fp32", 3, 17, 2, 64, True, 0),
    ("fp32", 1, 64, 3, 128, False, 0),
    ("bf16", 1, 3, 1, 64, True, 0),        # shorter than the filter
    ("fp32", 1, 41, 2, 64, True, 7),
    # head blocks of four heads: 2 and 8 (four and one token streams of workgroups, some past the last
    # token block), 3 and 5 (the plain numbering); ragged and packed token counts
    ("bf16", 2, 150, 8, 128, True, 0),
    ("bf16", 1, 500, 12, 64, True, 9),
    ("fp32", 1, 97, 32, 64, False, 4),
    ("bf16", 3, 65, 20, 64, True, 0),
])
def test_short_conv_matches_oracle(gdn, dtype, B, T, H, hd, l2, packed):
    flush(f"short conv {dtype} B={B} T={T} H={H} hd={hd} l2={l2} packed={packed}")
    inp = make_conv(B, T, H, hd, dtype, seed=T + H, num_packed=packed)
    cu = inp["cu_seqlens"]
    y = gdn.short_conv(inp["x"].cuda(), inp["w"].cuda(), cu_seqlens=cu.cuda() if cu is not None else None,
                       l2norm=l2, eps=1e-6)
    ref = oracle_conv(inp["x"], inp["w"], cu_seqlens=cu, l2norm=l2, eps=1e-6)
    assert_close("y", f64(y), ref, TOL[DT[dtype]])


def test_short_conv_b4_t4096_qk_shape(gdn):
    """q/k of prefill_b4_t4096 (4 x 4096 tokens, 16 heads x 128), L2-normalised: every element against the
    oracle, as a whole tensor and per (token, head) row."""
    flush("short conv full 4x4096x16x128")
    inp = make_conv(4, 4096, 16, 128, "bf16", seed=0)
    y = gdn.short_conv(inp["x"].cuda(), inp["w"].cuda(), l2norm=True)
    torch.cuda.synchronize()
    got = f64(y)
    ref = oracle_conv(inp["x"], inp["w"], l2norm=True)
    tol = TOL[torch.bfloat16]
    err = assert_close("y", got, ref, tol)
    per_row = np.sqrt(((got - ref) ** 2).sum(-1) / np.maximum((ref ** 2).sum(-1), 1e-300))
    flush(f"  rel-L2 {err:.2e}, worst row {per_row.max():.2e}")
    assert per_row.max() <= tol

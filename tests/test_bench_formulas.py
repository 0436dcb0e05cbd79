"""The algorithmic work and bytes bench.py divides by its measured times (the roofline fractions),
re-derived here a different way: the flops by listing every product of one chunk with its
dimensions, the bytes by adding up each tensor of the workload.  CPU only."""

import bench

from linear_attention_token_chunked_amd.inputs import WORKLOADS


def _chunk_products(Hqk, Hv, dk, dv, C):
    """(heads, m, n, k) of every dense tile product of one chunk of the chunked form."""
    return [
        (Hqk, C, C, dk),   # K K^T
        (Hqk, C, C, dk),   # Q K^T
        (Hv, C, dk, C),    # T K  (the solve, as a dense product with T = (I + A)^-1)
        (Hv, C, dv, C),    # T V
        (Hv, C, dv, C),    # P U
        (Hv, C, dv, dk),   # W M
        (Hv, C, dv, dk),   # Q M
        (Hv, dk, dv, C),   # K^T U  (the state update)
    ]


def test_prefill_flops_are_the_chunk_products():
    for Hqk, Hv, d, C in [(16, 16, 128, 64), (16, 32, 128, 64), (2, 4, 64, 64), (1, 3, 32, 16)]:
        per_chunk = sum(2 * h * m * n * k for h, m, n, k in _chunk_products(Hqk, Hv, d, d, C))
        assert bench.prefill_flops_per_token(Hqk, Hv, d, d, C) * C == per_chunk


def test_prefill_flops_per_launch_of_the_headline():
    w = WORKLOADS["varlen_64"]
    tokens = 210119  # the packed lengths of seed 0
    assert bench.prefill_flops_per_token(w.Hqk, w.Hv, w.dk, w.dv, w.chunk) * tokens == 1_101_628_702_720
    w1 = WORKLOADS["prefill_b4_t4096"]
    assert bench.prefill_flops_per_token(w1.Hqk, w1.Hv, w1.dk, w1.dv, w1.chunk) * w1.B * w1.T == 47_244_640_256


def test_prefill_bytes_are_the_tensors():
    w = WORKLOADS["prefill_b4_t4096"]
    tokens, s = w.B * w.T, 2
    q = k = tokens * w.Hqk * w.dk * s
    v = o = tokens * w.Hv * w.dv * s
    g = beta = tokens * w.Hv * 4
    states = 2 * w.B * w.Hv * w.dk * w.dv * 4  # initial state read, final state written
    assert bench.prefill_bytes(tokens, w.B, w.Hqk, w.Hv, w.dk, w.dv, s, True, True) == q + k + v + o + g + beta + states


def test_decode_and_verify_bytes():
    w = WORKLOADS["decode_n256"]
    state = w.N * w.Hv * w.dk * w.dv * 4
    token = w.N * (w.Hqk * w.dk * 2 * 2 + w.Hv * w.dv * 2 * 2 + w.Hv * 4 * 2)  # q, k; v, o; g, beta
    assert bench.decode_bytes(w.N, w.Hqk, w.Hv, w.dk, w.dv, 2) == 2 * state + token == 1_080_098_816
    wv = WORKLOADS["verify_n256_t4"]
    assert bench.verify_bytes(wv.N, wv.steps, wv.Hqk, wv.Hv, wv.dk, wv.dv, 2) == 2 * state + wv.steps * token
    assert bench.verify_bytes(wv.N, wv.steps, wv.Hqk, wv.Hv, wv.dk, wv.dv, 2) == 1_099_169_792


def test_bwd_bytes_are_the_tensors():
    w = WORKLOADS["prefill_b4_t4096"]
    tokens = w.B * w.T
    reads = tokens * (2 * w.Hqk * w.dk * 2 + 2 * w.Hv * w.dv * 2 + 2 * w.Hv * 4)  # q, k; v, dO; g, beta
    writes = tokens * (2 * w.Hqk * w.dk * 4 + w.Hv * w.dv * 4 + 2 * w.Hv * 4)     # dq, dk; dv; dg, dbeta
    states = 3 * w.B * w.Hv * w.dk * w.dv * 4  # initial state and d(final) read, d(initial) written
    assert bench.bwd_bytes(tokens, w.B, w.Hqk, w.Hv, w.dk, w.dv, 2) == reads + writes + states == 687_865_856

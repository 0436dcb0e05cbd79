"""C ABI checks that need no GPU: the library loads, exports every function the
header declares, and rejects invalid arguments before making any HIP call."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")
LIB = os.path.join(ROOT, "linear_attention_token_chunked_amd", "libgdn.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libgdn.so not built (run __graft_entry__.build())")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(gdn_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_ten_entry_points():
    assert declared_functions() == sorted(
        ["gdn_bwd_chunked", "gdn_bwd_chunked_workspace_size", "gdn_decode_step", "gdn_decode_verify",
         "gdn_fwd_chunked", "gdn_fwd_chunked_noalloc", "gdn_fwd_chunked_workspace_size", "gdn_output_norm_gate",
         "gdn_short_conv", "gdn_status_string"])


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(LIB)
    for name in declared_functions():
        assert hasattr(lib, name), name


@pytest.fixture(scope="module")
def gdn():
    from linear_attention_token_chunked_amd import gdn as m

    return m


def dims(gdn, **kw):
    base = dict(B=1, T=128, N=1, Hqk=2, Hv=4, dk=128, dv=128, chunk_size=64, scale=1.0)
    base.update(kw)
    dtype = kw.pop("dtype", None)
    import torch

    d = gdn.make_dims(base["B"], base["T"], base["N"], base["Hqk"], base["Hv"], base["dk"], base["dv"],
                      base["chunk_size"], base["scale"], torch.bfloat16)
    if dtype is not None:
        d.dtype = dtype
    return d


FAKE = 1 << 20  # an aligned, never-dereferenced address: validation must reject before using it


def call_fwd(gdn, d, q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, h0=0, cu=0, o=FAKE, hT=0, ws=0, ws_bytes=0):
    P = ctypes.c_void_p
    return gdn.lib.gdn_fwd_chunked(ctypes.byref(d), P(q), P(k), P(v), P(g), P(beta), P(h0), P(cu), P(o), P(hT), P(ws),
                                   ctypes.c_size_t(ws_bytes), P(0))


def call_noalloc(gdn, d, q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, h0=0, cu=0, o=FAKE, hT=0):
    P = ctypes.c_void_p
    return gdn.lib.gdn_fwd_chunked_noalloc(ctypes.byref(d), P(q), P(k), P(v), P(g), P(beta), P(h0), P(cu), P(o),
                                           P(hT), P(0))


def test_noalloc_validates_like_the_workspace_entry_point(gdn):
    """Invalid calls are rejected before any HIP call, with the statuses of gdn_fwd_chunked; the static
    scratch orders at most 4096 packed sequences, and more are rejected as too large for it."""
    assert call_noalloc(gdn, dims(gdn, Hv=3)) == INVALID
    assert call_noalloc(gdn, dims(gdn, chunk_size=32)) == NOT_SUPPORTED
    assert call_noalloc(gdn, dims(gdn), q=0) == INVALID
    assert call_noalloc(gdn, dims(gdn), q=FAKE + 8) == MISALIGNED
    assert call_noalloc(gdn, dims(gdn, B=2, N=2), cu=FAKE) == INVALID
    assert call_noalloc(gdn, dims(gdn, B=1, T=9000, N=4097, Hqk=1, Hv=1), cu=FAKE) == WORKSPACE_TOO_SMALL
    assert call_noalloc(gdn, dims(gdn, B=0, N=0)) == 0


def call_dec(gdn, d, q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, state=FAKE, o=FAKE):
    P = ctypes.c_void_p
    return gdn.lib.gdn_decode_step(ctypes.byref(d), P(q), P(k), P(v), P(g), P(beta), P(state), P(o), P(0))


def call_ver(gdn, d, q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, s_in=FAKE, s_out=0, ts=0, o=FAKE):
    P = ctypes.c_void_p
    return gdn.lib.gdn_decode_verify(ctypes.byref(d), P(q), P(k), P(v), P(g), P(beta), P(s_in), P(s_out), P(ts), P(o),
                                     P(0))


def call_bwd(gdn, d, q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, h0=0, cu=0, do=FAKE, dhT=0, dq=FAKE, dk=FAKE,
             dv=FAKE, dg=FAKE, dbeta=FAKE, dh0=0, ws=FAKE, ws_bytes=None):
    P = ctypes.c_void_p
    if ws_bytes is None:
        ws_bytes = gdn.bwd_chunked_workspace_size(d)
    return gdn.lib.gdn_bwd_chunked(ctypes.byref(d), P(q), P(k), P(v), P(g), P(beta), P(h0), P(cu), P(do), P(dhT),
                                   P(dq), P(dk), P(dv), P(dg), P(dbeta), P(dh0), P(ws), ctypes.c_size_t(ws_bytes),
                                   P(0))


INVALID, NOT_SUPPORTED, MISALIGNED, WORKSPACE_TOO_SMALL = 1, 2, 3, 4


def test_status_strings(gdn):
    for code in range(6):
        assert gdn.status_string(code).startswith("GDN_STATUS_")
    assert gdn.status_string(77) == "GDN_STATUS_UNKNOWN"


def test_null_dims_rejected(gdn):
    P = ctypes.c_void_p
    assert gdn.lib.gdn_fwd_chunked(None, P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(0), P(0), P(FAKE), P(0),
                                   P(0), ctypes.c_size_t(0), P(0)) == INVALID
    assert gdn.lib.gdn_decode_step(None, P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE),
                                   P(0)) == INVALID
    assert gdn.lib.gdn_fwd_chunked_workspace_size(None) == 0
    assert gdn.lib.gdn_decode_verify(None, P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(0), P(0), P(FAKE),
                                     P(0)) == INVALID


@pytest.mark.parametrize("kw,code", [
    (dict(Hv=3), INVALID),                 # Hv not a multiple of Hqk
    (dict(Hqk=0), INVALID),
    (dict(N=2), INVALID),                  # N != B without cu_seqlens
    (dict(T=-1), INVALID),
    (dict(dk=96, dv=96), NOT_SUPPORTED),   # head dims not built
    (dict(dk=128, dv=64), NOT_SUPPORTED),  # prefill needs dk == dv
    (dict(chunk_size=32), NOT_SUPPORTED),
    (dict(Hqk=1, Hv=8192), NOT_SUPPORTED),  # token rows beyond the kernels' 32-bit offsets
    (dict(dtype=7), INVALID),
])
def test_fwd_invalid_dims(gdn, kw, code):
    assert call_fwd(gdn, dims(gdn, **kw)) == code


def test_fwd_fp32_needs_dk64(gdn):
    d = dims(gdn, dtype=0)
    assert call_fwd(gdn, d) == NOT_SUPPORTED


def test_fwd_null_and_misaligned_pointers(gdn):
    d = dims(gdn)
    assert call_fwd(gdn, d, q=0) == INVALID
    assert call_fwd(gdn, d, o=0) == INVALID
    assert call_fwd(gdn, d, g=0) == INVALID
    assert call_fwd(gdn, d, v=FAKE + 8) == MISALIGNED
    assert call_fwd(gdn, d, hT=FAKE + 4) == MISALIGNED
    assert call_fwd(gdn, d, beta=FAKE + 2) == MISALIGNED


def test_fwd_cu_seqlens_requires_batch_one(gdn):
    d = dims(gdn, B=2, N=3)
    assert call_fwd(gdn, d, cu=FAKE) == INVALID


def test_fwd_empty_work_is_a_no_op_success(gdn):
    # zero sequences: nothing to launch, so success without touching the device
    assert call_fwd(gdn, dims(gdn, B=0, N=0)) == 0


def test_decode_invalid(gdn):
    assert call_dec(gdn, dims(gdn, T=2)) == INVALID           # one token per step
    assert call_dec(gdn, dims(gdn, B=2, N=3, T=1)) == INVALID  # batch must equal N
    assert call_dec(gdn, dims(gdn, T=1, Hv=5)) == INVALID
    assert call_dec(gdn, dims(gdn, T=1, dk=32)) == NOT_SUPPORTED
    assert call_dec(gdn, dims(gdn, T=1), state=0) == INVALID
    assert call_dec(gdn, dims(gdn, T=1), state=FAKE + 4) == MISALIGNED
    assert call_dec(gdn, dims(gdn, T=1, B=0, N=0)) == 0


def test_workspace_size_is_zero_for_the_fused_prefill(gdn):
    assert gdn.fwd_chunked_workspace_size(dims(gdn)) == 0
    # rows that fill the chip with their own units, short rows, fp32 and d = 64 run fused
    assert gdn.fwd_chunked_workspace_size(dims(gdn, B=4, T=4096, N=4, Hqk=16, Hv=16)) == 0
    assert gdn.fwd_chunked_workspace_size(dims(gdn, B=1, T=65536, N=1, Hqk=16, Hv=52)) == 0
    assert gdn.fwd_chunked_workspace_size(dims(gdn, T=3071, Hv=1, Hqk=1)) == 0
    assert gdn.fwd_chunked_workspace_size(dims(gdn, T=8192, dk=64, dv=64, dtype=0)) == 0
    assert gdn.fwd_chunked_workspace_size(dims(gdn, T=8192, dk=64, dv=64)) == 0


def test_packed_sequences_workspace(gdn):
    # packed sequences (batch 1, N > 1): N int32 for their longest-first order, up to 4096 sequences
    assert gdn.fwd_chunked_workspace_size(dims(gdn, B=1, T=1000, N=2)) == 256
    assert gdn.fwd_chunked_workspace_size(dims(gdn, B=1, T=1000, N=64)) == 256
    assert gdn.fwd_chunked_workspace_size(dims(gdn, B=1, T=1000, N=65)) == 512
    assert gdn.fwd_chunked_workspace_size(dims(gdn, B=1, T=0, N=4096)) == 16384
    assert gdn.fwd_chunked_workspace_size(dims(gdn, B=1, T=1000, N=4097)) == 0
    assert gdn.fwd_chunked_workspace_size(dims(gdn, B=1, T=1000, N=64, dk=64, dv=64, dtype=0)) == 256
    d = dims(gdn, B=1, T=1000, N=64)
    assert call_fwd(gdn, d, cu=FAKE, ws_bytes=255) == WORKSPACE_TOO_SMALL


def seg_ws_bytes(B, T, Hv, nseg):
    """Segmented prefill workspace: per-token bf16 vectors scale Phi_t^T q_t, then per segment and
    value head the zero-start end state and the transition (fp32), the start state (bf16, for the
    correction), and two fp32 states for the scan; each part padded to 256 bytes."""
    al = lambda x: (x + 255) // 256 * 256
    mat = 128 * 128
    return (al(B * T * Hv * 128 * 2) + 2 * al(nseg * B * Hv * mat * 4) + al(nseg * B * Hv * mat * 2)
            + 2 * al(B * Hv * mat * 4))


def test_segmented_prefill_workspace(gdn):
    # B = 1, T = 65536, 32 value heads: four segments (7 runs per head fill 224 of 256 compute units)
    d = dims(gdn, B=1, T=65536, N=1, Hqk=16, Hv=32)
    assert gdn.fwd_chunked_workspace_size(d) == seg_ws_bytes(1, 65536, 32, 4)
    # one head: at most T / 1024 segments, and none of them empty
    assert gdn.fwd_chunked_workspace_size(dims(gdn, T=3072, Hv=1, Hqk=1)) == seg_ws_bytes(1, 3072, 1, 3)
    assert gdn.fwd_chunked_workspace_size(dims(gdn, T=5000, Hv=1, Hqk=1)) == seg_ws_bytes(1, 5000, 1, 4)
    assert gdn.fwd_chunked_workspace_size(dims(gdn, B=1, T=65536, N=1, Hqk=1, Hv=51)) == seg_ws_bytes(1, 65536, 51, 3)
    need = gdn.fwd_chunked_workspace_size(d)
    assert call_fwd(gdn, d, ws_bytes=need - 1) == WORKSPACE_TOO_SMALL
    assert call_fwd(gdn, d, ws=FAKE + 128, ws_bytes=need) == MISALIGNED


def test_needed_workspace_must_be_given(gdn):
    """A declared size is not a buffer: with a workspace needed, a NULL one is rejected, whatever
    workspace_bytes says (no silent path without it)."""
    for d, cu in ((dims(gdn, B=1, T=65536, N=1, Hqk=16, Hv=32), 0), (dims(gdn, B=1, T=1000, N=64), FAKE)):
        need = gdn.fwd_chunked_workspace_size(d)
        assert need > 0
        assert call_fwd(gdn, d, cu=cu, ws=0, ws_bytes=need) == INVALID
        assert call_fwd(gdn, d, cu=cu, ws=0, ws_bytes=1 << 40) == INVALID


def test_one_packed_sequence_is_a_batch_row(gdn):
    """cu_seqlens with N = 1 is, by its contract {0, T}, the single batch row: the size query (which cannot
    see cu_seqlens) and the call agree on the same workspace, and that workspace is required."""
    row = dims(gdn, B=1, T=65536, N=1, Hqk=16, Hv=32)
    need = gdn.fwd_chunked_workspace_size(row)
    assert need > 0
    assert call_fwd(gdn, row, cu=FAKE, ws_bytes=need - 1) == WORKSPACE_TOO_SMALL
    assert call_fwd(gdn, row, cu=FAKE, ws=0, ws_bytes=need) == INVALID


def test_verify_invalid(gdn):
    assert call_ver(gdn, dims(gdn, T=0)) == INVALID              # at least one token
    assert call_ver(gdn, dims(gdn, T=9)) == NOT_SUPPORTED        # at most eight
    assert call_ver(gdn, dims(gdn, B=2, N=3, T=4)) == INVALID     # batch must equal N
    assert call_ver(gdn, dims(gdn, T=4, Hv=5)) == INVALID
    assert call_ver(gdn, dims(gdn, T=4, dk=32)) == NOT_SUPPORTED
    assert call_ver(gdn, dims(gdn, T=4), s_in=0) == INVALID
    assert call_ver(gdn, dims(gdn, T=4), o=0) == INVALID
    assert call_ver(gdn, dims(gdn, T=4), s_out=FAKE + 4) == MISALIGNED
    assert call_ver(gdn, dims(gdn, T=4), ts=FAKE + 8) == MISALIGNED
    assert call_ver(gdn, dims(gdn, T=4, B=0, N=0)) == 0          # nothing to do


def test_norm_gate_invalid(gdn):
    P = ctypes.c_void_p
    f = lambda rows=4, dv=128, eps=1e-6, dt=1, o=FAKE, z=FAKE, w=FAKE, y=FAKE: gdn.lib.gdn_output_norm_gate(
        ctypes.c_int64(rows), ctypes.c_int32(dv), ctypes.c_float(eps), dt, P(o), P(z), P(w), P(y), P(0))
    assert f(rows=-1) == INVALID
    assert f(eps=-1.0) == INVALID
    assert f(eps=float("nan")) == INVALID
    assert f(dt=5) == INVALID
    assert f(dv=96) == NOT_SUPPORTED
    assert f(o=0) == INVALID
    assert f(w=0) == INVALID
    assert f(z=FAKE + 8) == MISALIGNED
    assert f(w=FAKE + 4) == MISALIGNED
    assert f(rows=0) == 0                                          # nothing to do


def test_short_conv_invalid(gdn):
    P = ctypes.c_void_p
    f = lambda B=1, T=8, N=1, cu=0, H=2, hd=128, l2=1, eps=1e-6, dt=1, x=FAKE, w=FAKE, y=FAKE + 4096: \
        gdn.lib.gdn_short_conv(B, T, N, P(cu), H, hd, l2, ctypes.c_float(eps), dt, P(x), P(w), P(y), P(0))
    assert f(T=-1) == INVALID
    assert f(H=0) == INVALID
    assert f(B=2, N=3) == INVALID                       # N != B without cu_seqlens
    assert f(B=2, N=2, cu=FAKE) == INVALID              # packed input needs B == 1
    assert f(hd=96) == NOT_SUPPORTED
    assert f(eps=-1.0) == INVALID
    assert f(x=0) == INVALID
    assert f(y=FAKE) == INVALID                         # y must not be x
    assert f(w=FAKE + 4) == MISALIGNED
    assert f(T=0) == 0                                  # nothing to do


def bwd_ws_bytes(tokens, N, Hv, dk, dv, esize):
    al = lambda x: (x + 255) // 256 * 256
    chunks = tokens // 64 + N
    return al(4 * (N + 1)) + 2 * al(esize * chunks * Hv * dk * dv) + 2 * al(esize * tokens * Hv * dv)


def test_bwd_workspace_size(gdn):
    # chunk offsets, two states per value head and chunk, two values per token, head and channel,
    # in the element type of q, k, v
    assert gdn.bwd_chunked_workspace_size(dims(gdn, B=1, T=128, N=1)) == bwd_ws_bytes(128, 1, 4, 128, 128, 2)
    assert gdn.bwd_chunked_workspace_size(dims(gdn, B=3, T=100, N=3)) == bwd_ws_bytes(300, 3, 4, 128, 128, 2)
    assert gdn.bwd_chunked_workspace_size(dims(gdn, B=1, T=130, N=1, dk=64, dv=64, dtype=0)) == \
        bwd_ws_bytes(130, 1, 4, 64, 64, 4)
    assert gdn.lib.gdn_bwd_chunked_workspace_size(None) == 0
    # floor(total / 64) + N bounds the chunks of any split into N sequences
    for lens in ([1] * 7, [63, 65, 1], [64, 64], [0, 200, 0, 5]):
        chunks = sum(-(-n // 64) for n in lens)
        assert chunks <= sum(lens) // 64 + len(lens)


def test_bwd_invalid(gdn):
    assert call_bwd(gdn, dims(gdn, Hv=3)) == INVALID
    assert call_bwd(gdn, dims(gdn, N=2)) == INVALID                 # N != B without cu_seqlens
    assert call_bwd(gdn, dims(gdn, B=2, N=3), cu=FAKE) == INVALID   # packed input needs B == 1
    assert call_bwd(gdn, dims(gdn, dk=128, dv=64)) == NOT_SUPPORTED
    assert call_bwd(gdn, dims(gdn, chunk_size=32)) == NOT_SUPPORTED
    assert call_bwd(gdn, dims(gdn, dtype=0)) == NOT_SUPPORTED       # fp32 is built for dk = 64
    assert call_bwd(gdn, dims(gdn, dtype=7)) == INVALID
    assert call_bwd(gdn, dims(gdn), do=0) == INVALID
    assert call_bwd(gdn, dims(gdn), dg=0) == INVALID
    assert call_bwd(gdn, dims(gdn), dq=FAKE + 4) == MISALIGNED
    assert call_bwd(gdn, dims(gdn), dh0=FAKE + 8) == MISALIGNED
    assert call_bwd(gdn, dims(gdn), ws=FAKE + 64) == MISALIGNED
    d = dims(gdn)
    assert call_bwd(gdn, d, ws_bytes=gdn.bwd_chunked_workspace_size(d) - 1) == WORKSPACE_TOO_SMALL
    assert call_bwd(gdn, d, ws=0) == INVALID
    assert call_bwd(gdn, dims(gdn, B=0, N=0)) == 0                  # nothing to do

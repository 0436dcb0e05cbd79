"""Thin ctypes binding of libgdn.so (the C ABI in include/gdn.h).

Argument marshalling only: shapes and dtypes are checked, outputs are
allocated with torch on the inputs' device, and the call is enqueued on
torch's current HIP stream.  Every step of the mixer runs in the library's
gfx950 kernels; there is no other implementation behind these functions, and
importing this module fails loudly when the library has not been built.
"""

from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgdn.so")

STATUS_SUCCESS = 0


class Dims(ctypes.Structure):
    """Mirror of gdn_dims_t."""

    _fields_ = [
        ("batch", ctypes.c_int32),
        ("seqlen", ctypes.c_int32),
        ("num_seqs", ctypes.c_int32),
        ("num_qk_heads", ctypes.c_int32),
        ("num_v_heads", ctypes.c_int32),
        ("head_dim_k", ctypes.c_int32),
        ("head_dim_v", ctypes.c_int32),
        ("chunk_size", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("dtype", ctypes.c_int),
    ]


DTYPE_CODE = {torch.float32: 0, torch.bfloat16: 1}

EXPORTED = ("gdn_fwd_chunked_workspace_size", "gdn_fwd_chunked", "gdn_fwd_chunked_noalloc", "gdn_decode_step",
            "gdn_decode_verify",
            "gdn_output_norm_gate", "gdn_short_conv", "gdn_bwd_chunked_workspace_size", "gdn_bwd_chunked",
            "gdn_status_string")


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"{_LIB_PATH} is missing: build it first (python -m linear_attention_token_chunked_amd.build)")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, fp, sz = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t
    lib.gdn_fwd_chunked_workspace_size.argtypes = [ctypes.POINTER(Dims)]
    lib.gdn_fwd_chunked_workspace_size.restype = sz
    lib.gdn_fwd_chunked.argtypes = [ctypes.POINTER(Dims), vp, vp, vp, fp, fp, fp, vp, vp, fp, vp, sz, vp]
    lib.gdn_fwd_chunked.restype = ctypes.c_int
    lib.gdn_fwd_chunked_noalloc.argtypes = [ctypes.POINTER(Dims), vp, vp, vp, fp, fp, fp, vp, vp, fp, vp]
    lib.gdn_fwd_chunked_noalloc.restype = ctypes.c_int
    lib.gdn_decode_step.argtypes = [ctypes.POINTER(Dims), vp, vp, vp, fp, fp, fp, vp, vp]
    lib.gdn_decode_step.restype = ctypes.c_int
    lib.gdn_decode_verify.argtypes = [ctypes.POINTER(Dims), vp, vp, vp, fp, fp, fp, fp, fp, vp, vp]
    lib.gdn_decode_verify.restype = ctypes.c_int
    lib.gdn_output_norm_gate.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_int, vp, vp, fp, vp,
                                         vp]
    lib.gdn_output_norm_gate.restype = ctypes.c_int
    i32 = ctypes.c_int32
    lib.gdn_short_conv.argtypes = [i32, i32, i32, vp, i32, i32, i32, ctypes.c_float, ctypes.c_int, vp, fp, vp, vp]
    lib.gdn_short_conv.restype = ctypes.c_int
    lib.gdn_bwd_chunked_workspace_size.argtypes = [ctypes.POINTER(Dims)]
    lib.gdn_bwd_chunked_workspace_size.restype = sz
    lib.gdn_bwd_chunked.argtypes = [ctypes.POINTER(Dims), vp, vp, vp, fp, fp, fp, vp, vp, fp, fp, fp, fp, fp, fp, fp,
                                    vp, sz, vp]
    lib.gdn_bwd_chunked.restype = ctypes.c_int
    lib.gdn_status_string.argtypes = [ctypes.c_int]
    lib.gdn_status_string.restype = ctypes.c_char_p
    return lib


lib = _load()


def status_string(code: int) -> str:
    return lib.gdn_status_string(code).decode()


def _check(code: int):
    if code != STATUS_SUCCESS:
        raise RuntimeError(status_string(code))


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, name, dtype, device, ndim):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def make_dims(B, T, N, Hqk, Hv, dk, dv, chunk_size, scale, dtype) -> Dims:
    return Dims(B, T, N, Hqk, Hv, dk, dv, chunk_size, float(scale), DTYPE_CODE[dtype])


def fwd_chunked_workspace_size(dims: Dims) -> int:
    return int(lib.gdn_fwd_chunked_workspace_size(ctypes.byref(dims)))


def fwd_chunked(q, k, v, g, beta, *, initial_state=None, cu_seqlens=None, chunk_size=64, scale=1.0,
                output_final_state=True, out=None, final_state=None, workspace=None):
    """Chunked prefill: (o, final_state) for q, k [B, T, Hqk, dk], v [B, T, Hv, dv], g, beta [B, T, Hv].

    initial_state / final_state are fp32 [N, Hv, dk, dv]; cu_seqlens is int32 [N + 1] on the device
    (then B must be 1).  ``out`` and ``final_state`` may be given to reuse buffers; final_state may be
    the initial_state tensor itself for an in-place update.  ``workspace`` may be a uint8 device tensor
    of at least ``fwd_chunked_workspace_size`` bytes to reuse (long rows with few heads need one);
    otherwise one is allocated when needed.
    """
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU")
    _need(q, "q", q.dtype, dev, 4)
    if q.dtype not in DTYPE_CODE:
        raise TypeError("q, k, v must be float32 or bfloat16")
    B, T, Hqk, dk = q.shape
    _need(k, "k", q.dtype, dev, 4)
    _need(v, "v", q.dtype, dev, 4)
    Hv, dv = v.shape[2], v.shape[3]
    if k.shape != q.shape or v.shape[:2] != (B, T):
        raise ValueError("q, k, v shapes disagree")
    _need(g, "g", torch.float32, dev, 3)
    _need(beta, "beta", torch.float32, dev, 3)
    if g.shape != (B, T, Hv) or beta.shape != (B, T, Hv):
        raise ValueError("g and beta must be [B, T, Hv]")
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, dev, 1)
        N = cu_seqlens.shape[0] - 1
    else:
        N = B
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32, dev, 4)
        if initial_state.shape != (N, Hv, dk, dv):
            raise ValueError("initial_state must be [N, Hv, dk, dv]")
    if out is None:
        out = torch.empty((B, T, Hv, dv), dtype=q.dtype, device=dev)
    else:
        _need(out, "out", q.dtype, dev, 4)
        if out.shape != (B, T, Hv, dv):
            raise ValueError("out must be [B, T, Hv, dv]")
    if output_final_state and final_state is None:
        final_state = torch.empty((N, Hv, dk, dv), dtype=torch.float32, device=dev)
    if final_state is not None:
        _need(final_state, "final_state", torch.float32, dev, 4)
        if final_state.shape != (N, Hv, dk, dv):
            raise ValueError("final_state must be [N, Hv, dk, dv]")
    dims = make_dims(B, T, N, Hqk, Hv, dk, dv, chunk_size, scale, q.dtype)
    ws_bytes = fwd_chunked_workspace_size(dims)
    ws = workspace
    if ws is None:
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
    else:
        _need(ws, "workspace", torch.uint8, dev, 1)
        ws_bytes = ws.numel()
    with torch.cuda.device(dev):
        code = lib.gdn_fwd_chunked(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                   _ptr(initial_state), _ptr(cu_seqlens), _ptr(out), _ptr(final_state), _ptr(ws),
                                   ctypes.c_size_t(ws_bytes), _stream(dev))
    _check(code)
    return out, final_state


def fwd_chunked_noalloc(q, k, v, g, beta, *, initial_state=None, cu_seqlens=None, chunk_size=64, scale=1.0,
                        out, final_state=None):
    """fwd_chunked through gdn_fwd_chunked_noalloc: nothing is allocated, by the library or here.
    ``out`` [B, T, Hv, dv] is required; ``final_state`` [N, Hv, dk, dv] fp32 is written when given.
    Returns (out, final_state)."""
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU")
    if q.dtype not in DTYPE_CODE:
        raise TypeError("q, k, v must be float32 or bfloat16")
    _need(q, "q", q.dtype, dev, 4)
    B, T, Hqk, dk = q.shape
    _need(k, "k", q.dtype, dev, 4)
    _need(v, "v", q.dtype, dev, 4)
    Hv, dv = v.shape[2], v.shape[3]
    if k.shape != q.shape or v.shape[:2] != (B, T):
        raise ValueError("q, k, v shapes disagree")
    _need(g, "g", torch.float32, dev, 3)
    _need(beta, "beta", torch.float32, dev, 3)
    if g.shape != (B, T, Hv) or beta.shape != (B, T, Hv):
        raise ValueError("g and beta must be [B, T, Hv]")
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, dev, 1)
        N = cu_seqlens.shape[0] - 1
    else:
        N = B
    for name, st in (("initial_state", initial_state), ("final_state", final_state)):
        if st is not None:
            _need(st, name, torch.float32, dev, 4)
            if st.shape != (N, Hv, dk, dv):
                raise ValueError(f"{name} must be [N, Hv, dk, dv]")
    _need(out, "out", q.dtype, dev, 4)
    if out.shape != (B, T, Hv, dv):
        raise ValueError("out must be [B, T, Hv, dv]")
    dims = make_dims(B, T, N, Hqk, Hv, dk, dv, chunk_size, scale, q.dtype)
    with torch.cuda.device(dev):
        code = lib.gdn_fwd_chunked_noalloc(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                           _ptr(initial_state), _ptr(cu_seqlens), _ptr(out), _ptr(final_state),
                                           _stream(dev))
    _check(code)
    return out, final_state


def decode_step(q, k, v, g, beta, state, *, scale=1.0, out=None):
    """One decode step for N sequences; updates ``state`` [N, Hv, dk, dv] fp32 in place, returns o [N, Hv, dv]."""
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU")
    if q.dtype not in DTYPE_CODE:
        raise TypeError("q, k, v must be float32 or bfloat16")
    _need(q, "q", q.dtype, dev, 3)
    N, Hqk, dk = q.shape
    _need(k, "k", q.dtype, dev, 3)
    _need(v, "v", q.dtype, dev, 3)
    Hv, dv = v.shape[1], v.shape[2]
    if k.shape != q.shape or v.shape[0] != N:
        raise ValueError("q, k, v shapes disagree")
    _need(g, "g", torch.float32, dev, 2)
    _need(beta, "beta", torch.float32, dev, 2)
    _need(state, "state", torch.float32, dev, 4)
    if g.shape != (N, Hv) or beta.shape != (N, Hv) or state.shape != (N, Hv, dk, dv):
        raise ValueError("g, beta must be [N, Hv] and state [N, Hv, dk, dv]")
    if out is None:
        out = torch.empty((N, Hv, dv), dtype=q.dtype, device=dev)
    else:
        _need(out, "out", q.dtype, dev, 3)
    dims = make_dims(N, 1, N, Hqk, Hv, dk, dv, 64, scale, q.dtype)
    with torch.cuda.device(dev):
        code = lib.gdn_decode_step(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state),
                                   _ptr(out), _stream(dev))
    _check(code)
    return out


def decode_verify(q, k, v, g, beta, state_in, *, state_out="in_place", token_states=None, scale=1.0, out=None):
    """Tv consecutive decode steps per sequence from ``state_in`` (multi-token verify).

    q, k [N, Tv, Hqk, dk], v [N, Tv, Hv, dv], g, beta [N, Tv, Hv], state_in [N, Hv, dk, dv] fp32.
    ``state_out``: "in_place" (default: state_in is updated), None (not written) or a tensor.
    ``token_states``: None, or an fp32 [N, Tv, Hv, dk, dv] tensor that receives the state after
    every token.  Returns o [N, Tv, Hv, dv].
    """
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU")
    if q.dtype not in DTYPE_CODE:
        raise TypeError("q, k, v must be float32 or bfloat16")
    _need(q, "q", q.dtype, dev, 4)
    N, Tv, Hqk, dk = q.shape
    _need(k, "k", q.dtype, dev, 4)
    _need(v, "v", q.dtype, dev, 4)
    Hv, dv = v.shape[2], v.shape[3]
    if k.shape != q.shape or v.shape[:2] != (N, Tv):
        raise ValueError("q, k, v shapes disagree")
    _need(g, "g", torch.float32, dev, 3)
    _need(beta, "beta", torch.float32, dev, 3)
    if g.shape != (N, Tv, Hv) or beta.shape != (N, Tv, Hv):
        raise ValueError("g, beta must be [N, Tv, Hv]")
    _need(state_in, "state_in", torch.float32, dev, 4)
    if state_in.shape != (N, Hv, dk, dv):
        raise ValueError("state_in must be [N, Hv, dk, dv]")
    if isinstance(state_out, str):
        if state_out != "in_place":
            raise ValueError('state_out must be "in_place", None or a tensor')
        state_out = state_in
    if state_out is not None:
        _need(state_out, "state_out", torch.float32, dev, 4)
        if state_out.shape != (N, Hv, dk, dv):
            raise ValueError("state_out must be [N, Hv, dk, dv]")
    if token_states is not None:
        _need(token_states, "token_states", torch.float32, dev, 5)
        if token_states.shape != (N, Tv, Hv, dk, dv):
            raise ValueError("token_states must be [N, Tv, Hv, dk, dv]")
    if out is None:
        out = torch.empty((N, Tv, Hv, dv), dtype=q.dtype, device=dev)
    else:
        _need(out, "out", q.dtype, dev, 4)
        if out.shape != (N, Tv, Hv, dv):
            raise ValueError("out must be [N, Tv, Hv, dv]")
    dims = make_dims(N, Tv, N, Hqk, Hv, dk, dv, 64, scale, q.dtype)
    with torch.cuda.device(dev):
        code = lib.gdn_decode_verify(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                     _ptr(state_in), _ptr(state_out), _ptr(token_states), _ptr(out), _stream(dev))
    _check(code)
    return out


def output_norm_gate(o, z, weight, *, eps=1e-6, out=None):
    """y = sigmoid(z) * o / sqrt(mean(o^2) + eps) * (1 + weight) over the last dim (dv) of o.

    o, z: contiguous tensors of the same shape [..., dv] (fp32 or bf16); weight: fp32 [dv].
    ``out`` may be ``o`` itself (in place).  Returns y.
    """
    dev = o.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU")
    if o.dtype not in DTYPE_CODE:
        raise TypeError("o, z must be float32 or bfloat16")
    if o.dim() < 1:
        raise ValueError("o must have a last (dv) dimension")
    _need(o, "o", o.dtype, dev, o.dim())
    _need(z, "z", o.dtype, dev, o.dim())
    if z.shape != o.shape:
        raise ValueError("z must have the shape of o")
    dv = o.shape[-1]
    _need(weight, "weight", torch.float32, dev, 1)
    if weight.shape[0] != dv:
        raise ValueError("weight must be [dv]")
    if out is None:
        out = torch.empty_like(o)
    else:
        _need(out, "out", o.dtype, dev, o.dim())
        if out.shape != o.shape:
            raise ValueError("out must have the shape of o")
    rows = o.numel() // dv if dv else 0
    with torch.cuda.device(dev):
        code = lib.gdn_output_norm_gate(ctypes.c_int64(rows), ctypes.c_int32(dv), ctypes.c_float(eps),
                                        DTYPE_CODE[o.dtype], _ptr(o), _ptr(z), _ptr(weight), _ptr(out), _stream(dev))
    _check(code)
    return out


SHORT_CONV_WIDTH = 4


def short_conv(x, weight, *, cu_seqlens=None, l2norm=False, eps=1e-6, out=None):
    """Short causal convolution (width 4) along the tokens of x [B, T, heads, head_dim], per
    channel, restarting at every sequence start; then, with ``l2norm``, every (token, head) row
    scaled to unit L2 norm.  weight: fp32 [heads * head_dim, 4], tap i multiplying token t - 3 + i.
    cu_seqlens: int32 [N + 1] on the device (then B must be 1), or None.  Returns y (a new tensor,
    or ``out``, which must not be x)."""
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU")
    if x.dtype not in DTYPE_CODE:
        raise TypeError("x must be float32 or bfloat16")
    _need(x, "x", x.dtype, dev, 4)
    B, T, H, hd = x.shape
    _need(weight, "weight", torch.float32, dev, 2)
    if weight.shape != (H * hd, SHORT_CONV_WIDTH):
        raise ValueError("weight must be [heads * head_dim, 4]")
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, dev, 1)
        N = cu_seqlens.shape[0] - 1
    else:
        N = B
    if out is None:
        out = torch.empty_like(x)
    else:
        _need(out, "out", x.dtype, dev, 4)
        if out.shape != x.shape:
            raise ValueError("out must have the shape of x")
    with torch.cuda.device(dev):
        code = lib.gdn_short_conv(B, T, N, _ptr(cu_seqlens), H, hd, int(bool(l2norm)), ctypes.c_float(eps),
                                  DTYPE_CODE[x.dtype], _ptr(x), _ptr(weight), _ptr(out), _stream(dev))
    _check(code)
    return out


def bwd_chunked_workspace_size(dims: Dims) -> int:
    return int(lib.gdn_bwd_chunked_workspace_size(ctypes.byref(dims)))


def bwd_chunked(q, k, v, g, beta, d_o, *, initial_state=None, d_final_state=None, cu_seqlens=None, chunk_size=64,
                scale=1.0, want_d_initial_state=True, workspace=None):
    """Backward of ``fwd_chunked``: a dict of fp32 gradients dq, dk [B, T, Hqk, dk], dv [B, T, Hv, dv],
    dg, dbeta [B, T, Hv] and d_initial_state [N, Hv, dk, dv] (None unless ``want_d_initial_state``).

    The inputs are those of the forward pass; ``d_o`` [B, T, Hv, dv] has q's dtype and
    ``d_final_state`` is fp32 [N, Hv, dk, dv] or None.  ``workspace`` may be a uint8 device tensor of
    at least ``bwd_chunked_workspace_size`` bytes to reuse; otherwise one is allocated.
    """
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU")
    _need(q, "q", q.dtype, dev, 4)
    if q.dtype not in DTYPE_CODE:
        raise TypeError("q, k, v must be float32 or bfloat16")
    B, T, Hqk, dk = q.shape
    _need(k, "k", q.dtype, dev, 4)
    _need(v, "v", q.dtype, dev, 4)
    _need(d_o, "d_o", q.dtype, dev, 4)
    Hv, dv = v.shape[2], v.shape[3]
    if k.shape != q.shape or v.shape[:2] != (B, T) or d_o.shape != v.shape:
        raise ValueError("q, k, v, d_o shapes disagree")
    _need(g, "g", torch.float32, dev, 3)
    _need(beta, "beta", torch.float32, dev, 3)
    if g.shape != (B, T, Hv) or beta.shape != (B, T, Hv):
        raise ValueError("g and beta must be [B, T, Hv]")
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, dev, 1)
        N = cu_seqlens.shape[0] - 1
    else:
        N = B
    for name, st in (("initial_state", initial_state), ("d_final_state", d_final_state)):
        if st is not None:
            _need(st, name, torch.float32, dev, 4)
            if st.shape != (N, Hv, dk, dv):
                raise ValueError(f"{name} must be [N, Hv, dk, dv]")
    f32 = dict(dtype=torch.float32, device=dev)
    grads = {"dq": torch.empty((B, T, Hqk, dk), **f32), "dk": torch.empty((B, T, Hqk, dk), **f32),
             "dv": torch.empty((B, T, Hv, dv), **f32), "dg": torch.empty((B, T, Hv), **f32),
             "dbeta": torch.empty((B, T, Hv), **f32),
             "d_initial_state": torch.empty((N, Hv, dk, dv), **f32) if want_d_initial_state else None}
    dims = make_dims(B, T, N, Hqk, Hv, dk, dv, chunk_size, scale, q.dtype)
    ws_bytes = bwd_chunked_workspace_size(dims)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    else:
        _need(workspace, "workspace", torch.uint8, dev, 1)
    with torch.cuda.device(dev):
        code = lib.gdn_bwd_chunked(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                   _ptr(initial_state), _ptr(cu_seqlens), _ptr(d_o), _ptr(d_final_state),
                                   _ptr(grads["dq"]), _ptr(grads["dk"]), _ptr(grads["dv"]), _ptr(grads["dg"]),
                                   _ptr(grads["dbeta"]), _ptr(grads["d_initial_state"]), _ptr(workspace),
                                   ctypes.c_size_t(workspace.numel()), _stream(dev))
    _check(code)
    return grads

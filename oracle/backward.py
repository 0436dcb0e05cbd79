"""fp64 CPU oracle for the backward pass of the GDN token mixer.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: imported by tests/ and
never by the product path.

The gradients are those of the scalar  sum(o * d_o) + sum(final_state * d_final)
with respect to q, k, v, g, beta and the initial state, for the recurrence of
``oracle.recurrent`` (podcast transcript on "On the Design of Qwen3.8-Next
Architecture", cue 14: decay, read under the key, write the error).  The
recurrence is written out again token by token with plain PyTorch CPU ops in
float64, and torch's reverse-mode automatic differentiation forms the
gradients: nothing here derives or transcribes an adjoint by hand, so the GPU
backward (a hand-derived adjoint) shares no reasoning with it.  Its own pins
compare it with central finite differences of ``oracle.recurrent``.
"""

from __future__ import annotations

import numpy as np
import torch

from .gdn_oracle import _f64, sequence_bounds


def recurrent_grads(q, k, v, g, beta, d_o, initial_state=None, d_final=None, cu_seqlens=None, scale=1.0):
    """Returns a dict of float64 numpy arrays: dq, dk [B, T, Hqk, dk]; dv [B, T, Hv, dv];
    dg, dbeta [B, T, Hv]; d_initial_state [N, Hv, dk, dv] (zeros' gradient if initial_state is None)."""
    t = lambda x: torch.tensor(_f64(x), dtype=torch.float64)
    q, k, v, g, beta, d_o = (t(x) for x in (q, k, v, g, beta, d_o))
    B, T, Hqk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    head_of = torch.arange(Hv) // (Hv // Hqk)
    seqs = sequence_bounds(B, T, cu_seqlens)
    S0 = t(initial_state) if initial_state is not None else torch.zeros((len(seqs), Hv, dk, dv), dtype=torch.float64)
    for x in (q, k, v, g, beta, S0):
        x.requires_grad_(True)
    loss = torch.zeros((), dtype=torch.float64)
    for n, (b, s, e) in enumerate(seqs):
        M = S0[n]
        for tok in range(s, e):
            alpha = torch.exp(g[b, tok])                     # [Hv]
            kt = k[b, tok, head_of]                          # [Hv, dk]
            qt = scale * q[b, tok, head_of]
            decayed = alpha[:, None, None] * M
            read = torch.einsum("hi,hij->hj", kt, decayed)
            M = decayed + beta[b, tok][:, None, None] * kt[:, :, None] * (v[b, tok] - read)[:, None, :]
            o_t = torch.einsum("hij,hi->hj", M, qt)
            loss = loss + (o_t * d_o[b, tok]).sum()
        if d_final is not None:
            loss = loss + (M * t(d_final)[n]).sum()
    loss.backward()
    grad = lambda x: x.grad.detach().numpy() if x.grad is not None else np.zeros(tuple(x.shape))
    return {"dq": grad(q), "dk": grad(k), "dv": grad(v), "dg": grad(g), "dbeta": grad(beta),
            "d_initial_state": grad(S0)}

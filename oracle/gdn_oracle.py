"""Plain fp64 CPU oracle for the Gated DeltaNet (GDN) token mixer.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The product path
(the HIP library ``libgdn.so`` and its Python binding) never imports, links or
calls anything here, and the two share no code.  Everything runs in float64 on
the host; inputs are upcast exactly (bf16 and fp32 values are representable in
fp64), so the oracle consumes the very values the GPU consumes.

What the method computes
------------------------
Source: podcast transcript "On the Design of Qwen3.8-Next Architecture"
(episode "Qwen3.8-Next design: hybrid attention, residuals and n-gram
embeddings"), cue 14, and cue 4 of the same transcript.  Cue 4: the GDN layers
compress the prefix into a state of fixed size, at a cost linear in the length.
Cue 14: each step, a decay alpha first shrinks the whole state; the rule then
reads what the state holds under the current key, subtracts that from the new
value and writes only the difference, so one key written twice leaves a single,
corrected entry.  Written out for one head, with the math-layout state S of
shape (dv, dk), decay alpha_t = exp(g_t) and write strength beta_t:

    S_t = alpha_t * S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
        = alpha_t * S_{t-1} + beta_t (v_t - alpha_t S_{t-1} k_t) k_t^T
    o_t = S_t q_t

The second line is the transcript's order of operations (decay, read under the
key, write the error); the first is the same map as a product of a transition
matrix and an input term.

Readings taken where the pages are silent (the HIP path takes the same ones)
----------------------------------------------------------------------------
R1  States are stored as M = S^T with shape (dk, dv): M[i, j] = S[j, i].  The
    update in this layout is M <- alpha (I - beta k k^T) M + beta k v^T and the
    output is o = M^T q.  Initial and final states use the same layout.
R2  o_t reads the state *after* token t's own write (o_t = S_t q_t).
R3  Decay is applied before the read: alpha S + beta (v - alpha S k) k^T.
R4  The gate is passed as g = log(alpha) (fp32); beta is passed after its
    sigmoid (fp32).
R5  q is multiplied by ``scale`` (1.0 reproduces o_t = S_t q_t exactly).
R6  With Hv value heads and Hqk query/key heads (Hv a multiple of Hqk), value
    head h reads query/key head h // (Hv // Hqk); g and beta are per value head.
R8  Chunks restart at every sequence start; a short last chunk is processed
    as it is (equivalent to padding with g = 0, beta = 0).
R9  Layouts: q, k [B, T, Hqk, dk]; v, o [B, T, Hv, dv]; g, beta [B, T, Hv];
    states [N, Hv, dk, dv].  Packed variable-length input uses B = 1 and
    cu_seqlens [N + 1] with cu[0] = 0 <= ... <= cu[N] = T.
R14 A missing initial state means zeros.
R15 Empty sequences are allowed; their final state equals their initial state.
R20 exp(G_i - G_j) is formed only for i >= j (the upper triangle can overflow).
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "recurrent",
    "chunked",
    "chunk_factors",
    "unrolled",
    "decode_step",
    "sequence_bounds",
]


def _f64(x):
    """Exact upcast of a numpy array or a CPU/GPU torch tensor to float64 numpy."""
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor (bf16 has no numpy dtype)
        import torch

        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def sequence_bounds(B, T, cu_seqlens=None):
    """List of (batch_row, start, end) for every sequence (reading R9).

    Without cu_seqlens every batch row is one sequence of length T.  With it,
    B must be 1 and sequence n covers tokens [cu[n], cu[n+1]).
    """
    if cu_seqlens is None:
        return [(b, 0, T) for b in range(B)]
    cu = np.asarray(cu_seqlens.cpu() if hasattr(cu_seqlens, "cpu") else cu_seqlens).astype(np.int64)
    if B != 1:
        raise ValueError("packed sequences need B == 1")
    if cu[0] != 0 or cu[-1] != T or np.any(np.diff(cu) < 0):
        raise ValueError("cu_seqlens must start at 0, end at T and not decrease")
    return [(0, int(cu[n]), int(cu[n + 1])) for n in range(len(cu) - 1)]


def _unpack(q, k, v, g, beta, initial_state, cu_seqlens):
    q, k, v, g, beta = (_f64(x) for x in (q, k, v, g, beta))
    B, T, Hqk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    if k.shape != q.shape or v.shape[:2] != (B, T) or g.shape != (B, T, Hv) or beta.shape != (B, T, Hv):
        raise ValueError("inconsistent shapes")
    if Hv % Hqk:
        raise ValueError("Hv must be a multiple of Hqk")
    head_of = np.arange(Hv) // (Hv // Hqk)  # reading R6
    seqs = sequence_bounds(B, T, cu_seqlens)
    S0 = _f64(initial_state)
    if S0 is not None and S0.shape != (len(seqs), Hv, dk, dv):
        raise ValueError("initial_state must be [N, Hv, dk, dv]")
    return q, k, v, g, beta, S0, head_of, seqs


def recurrent(q, k, v, g, beta, initial_state=None, cu_seqlens=None, scale=1.0):
    """Token-by-token gated delta rule, the definition itself.

    Follows the transcript's cue 14 step order for every token: decay the
    whole state, read what is stored under the key, write the error scaled by
    beta, then read the output from the updated state (R2, R3).  Returns
    (o [B, T, Hv, dv], final_state [N, Hv, dk, dv]) in float64.
    """
    q, k, v, g, beta, S0, head_of, seqs = _unpack(q, k, v, g, beta, initial_state, cu_seqlens)
    B, T, Hqk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    o = np.zeros((B, T, Hv, dv))
    final = np.zeros((len(seqs), Hv, dk, dv))
    for n, (b, s, e) in enumerate(seqs):
        M = S0[n].copy() if S0 is not None else np.zeros((Hv, dk, dv))
        for t in range(s, e):
            alpha = np.exp(g[b, t])  # [Hv]
            bt = beta[b, t]  # [Hv]
            kt = k[b, t, head_of]  # [Hv, dk]
            qt = scale * q[b, t, head_of]  # [Hv, dk]
            vt = v[b, t]  # [Hv, dv]
            decayed = alpha[:, None, None] * M  # alpha S
            read = np.einsum("hi,hij->hj", kt, decayed)  # (alpha S) k, as a dv-vector
            error = vt - read  # what the key should hold minus what it holds
            M = decayed + bt[:, None, None] * kt[:, :, None] * error[:, None, :]
            o[b, t] = np.einsum("hij,hi->hj", M, qt)  # S_t q_t
        final[n] = M
    return o, final


def decode_step(q, k, v, g, beta, state, scale=1.0):
    """One recurrent step for N independent sequences.

    q, k [N, Hqk, dk]; v [N, Hv, dv]; g, beta [N, Hv]; state [N, Hv, dk, dv].
    Returns (o [N, Hv, dv], new_state) in float64.  It is the recurrence above
    with T = 1 per sequence, the state read from and written back to ``state``.
    """
    q, k, v, g, beta, state = (_f64(x) for x in (q, k, v, g, beta, state))
    o, new_state = recurrent(q[:, None], k[:, None], v[:, None], g[:, None], beta[:, None],
                             initial_state=state, scale=scale)
    return o[:, 0], new_state


def verify(q, k, v, g, beta, state, scale=1.0):
    """Multi-token verify: Tv consecutive steps per sequence from a live state.

    Speculative decoding (the archdiff model page "Qwen3.8-2.4T-A95B",
    components list: multi-token-prediction drafting) runs every drafted token
    through the layer; here that is ``decode_step`` applied once per token, in
    order, each step starting from the state the previous one left.
    q, k [N, Tv, Hqk, dk]; v [N, Tv, Hv, dv]; g, beta [N, Tv, Hv]; state [N, Hv, dk, dv].
    Returns (o [N, Tv, Hv, dv], token_states [N, Tv, Hv, dk, dv]) in float64,
    token_states[:, t] being the state after token t (the last is the final state).
    """
    q, k, v, g, beta, state = (_f64(x) for x in (q, k, v, g, beta, state))
    N, Tv = q.shape[:2]
    o = np.zeros((N, Tv) + v.shape[2:])
    states = np.zeros((N, Tv) + state.shape[1:])
    for t in range(Tv):
        o[:, t], state = decode_step(q[:, t], k[:, t], v[:, t], g[:, t], beta[:, t], state, scale=scale)
        states[:, t] = state
    return o, states


def output_norm_gate(o, z, weight, eps=1e-6):
    """Output epilogue around the mixer, per row of dv values (the last axis).

    The podcast transcript (cue 14) adds a sigmoid output gate and a
    zero-centred RMSNorm to the rule; the archdiff model page "Qwen3.8-2.4T-A95B"
    writes the gate as sigmoid(x W_g) times o.  Readings (R21): the norm comes
    first and the gate multiplies its result; the norm divides by the root of
    the mean square over the row plus eps; "zero-centred" means the stored
    weight w scales by 1 + w.  z stands for the pre-activation x W_g.
    """
    o, z, weight = (_f64(x) for x in (o, z, weight))
    rms = np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
    gate = 1.0 / (1.0 + np.exp(-z))
    return gate * (o / rms) * (1.0 + weight)


def short_conv(x, weight, cu_seqlens=None, l2norm=False, eps=1e-6):
    """Pre-mixer short causal convolution along the tokens, per channel.

    The podcast transcript (cue 14) lists short causal convolutions around the
    rule without a width; the width here is that of ``weight`` (4 for the GPU
    path).  Readings (R23): tap i of W multiplies token t - (W - 1) + i, tokens
    before a sequence's start count as zero, there is no activation after it;
    with l2norm every (token, head) row is then divided by
    sqrt(sum of squares + eps) (the per-head q/k normalisation, to unit norm).
    x [B, T, heads, hd]; weight [heads * hd, W]; returns y in float64.
    """
    x, weight = _f64(x), _f64(weight)
    B, T, H, hd = x.shape
    W = weight.shape[1]
    wc = weight.reshape(H, hd, W)
    y = np.zeros_like(x)
    for b, s, e in sequence_bounds(B, T, cu_seqlens):
        for t in range(s, e):
            for i in range(W):
                u = t - (W - 1) + i
                if u >= s:
                    y[b, t] += wc[:, :, i] * x[b, u]
    if l2norm:
        y = y / np.sqrt(np.sum(y * y, axis=-1, keepdims=True) + eps)
    return y


def chunk_factors(K, V, g, beta):
    """Chunk-local factors of the chunked (UT / WY) form for one chunk.

    K [H, L, dk], V [H, L, dv], g, beta [H, L] (already per value head).
    Returns a dict with
      G   inclusive cumulative sum of g inside the chunk          [H, L]
      D   decay matrix exp(G_i - G_j) for i >= j, 0 above          [H, L, L]
      A   strict_tril(diag(beta) (D * K K^T))                      [H, L, L]
      T   (I + A)^-1                                                [H, L, L]
      W   T diag(beta * exp(G)) K                                   [H, L, dk]
      Ut  T diag(beta) V                                            [H, L, dv]
    Derivation (unrolling the recurrence inside a chunk that starts from state
    M): u_t = beta_t (v_t - exp(G_t) M^T k_t - sum_{s<t} exp(G_t - G_s) (k_t.k_s) u_s),
    i.e. (I + A) U = diag(beta) V - diag(beta exp(G)) K M, so U = Ut - W M.
    """
    H, L = g.shape
    G = np.cumsum(g, axis=1)
    low = np.tril(np.ones((L, L), dtype=bool))
    diff = np.where(low, G[:, :, None] - G[:, None, :], 0.0)  # R20: only i >= j
    D = np.where(low, np.exp(diff), 0.0)
    KK = K @ np.swapaxes(K, 1, 2)
    A = np.tril(beta[:, :, None] * D * KK, -1)
    eye = np.broadcast_to(np.eye(L), (H, L, L))
    T = np.linalg.solve(eye + A, eye)
    W = T @ ((beta * np.exp(G))[:, :, None] * K)
    Ut = T @ (beta[:, :, None] * V)
    return {"G": G, "D": D, "A": A, "T": T, "W": W, "Ut": Ut}


def chunked(q, k, v, g, beta, chunk_size, initial_state=None, cu_seqlens=None, scale=1.0):
    """The chunked-parallel form in float64, for any chunk size C >= 1.

    Per chunk and value head, with M the state entering the chunk:
      G, A, T, W, Ut from ``chunk_factors``
      U      = Ut - W M
      O      = diag(exp G) Q M + (D * Q K^T) U        (mask includes the diagonal, R2)
      M_next = exp(G_L) M + (diag(exp(G_L - G)) K)^T U
    Chunks restart at every sequence start; a short last chunk is processed as
    it is (R8).  Exact in real arithmetic; equals ``recurrent`` up to rounding.
    """
    if chunk_size < 1:
        raise ValueError("chunk_size must be >= 1")
    q, k, v, g, beta, S0, head_of, seqs = _unpack(q, k, v, g, beta, initial_state, cu_seqlens)
    B, T, Hqk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    o = np.zeros((B, T, Hv, dv))
    final = np.zeros((len(seqs), Hv, dk, dv))
    for n, (b, s, e) in enumerate(seqs):
        M = S0[n].copy() if S0 is not None else np.zeros((Hv, dk, dv))
        for c0 in range(s, e, chunk_size):
            c1 = min(c0 + chunk_size, e)
            K = np.swapaxes(k[b, c0:c1][:, head_of], 0, 1)  # [Hv, L, dk]
            Q = scale * np.swapaxes(q[b, c0:c1][:, head_of], 0, 1)
            V = np.swapaxes(v[b, c0:c1], 0, 1)  # [Hv, L, dv]
            gc = g[b, c0:c1].T  # [Hv, L]
            bc = beta[b, c0:c1].T
            f = chunk_factors(K, V, gc, bc)
            G, D = f["G"], f["D"]
            U = f["Ut"] - f["W"] @ M
            O = np.exp(G)[:, :, None] * (Q @ M) + (D * (Q @ np.swapaxes(K, 1, 2))) @ U
            o[b, c0:c1] = np.swapaxes(O, 0, 1)
            GL = G[:, -1:]
            Kt = np.exp(GL - G)[:, :, None] * K
            M = np.exp(GL)[:, :, None] * M + np.swapaxes(Kt, 1, 2) @ U
        final[n] = M
    return o, final


def unrolled(q, k, v, g, beta, initial_state=None, scale=1.0):
    """Brute-force closed form in math layout, for a single short sequence.

    With A_t = alpha_t (I - beta_t k_t k_t^T) (dk x dk) and S_0 = initial_state^T:
        S_t = S_0 A_1 A_2 ... A_t + sum_{s <= t} beta_s v_s k_s^T A_{s+1} ... A_t
        o_t = S_t q_t
    Every S_t is rebuilt from scratch from these explicit products (formed
    left to right in increasing t), so nothing is shared with ``recurrent``.
    Inputs use B = 1.  Returns (o [1, T, Hv, dv], final_state [1, Hv, dk, dv]).
    """
    q, k, v, g, beta = (_f64(x) for x in (q, k, v, g, beta))
    _, T, Hqk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    rep = Hv // Hqk
    S0 = _f64(initial_state)
    o = np.zeros((1, T, Hv, dv))
    final = np.zeros((1, Hv, dk, dv))
    I = np.eye(dk)
    for h in range(Hv):
        hq = h // rep
        S_init = S0[0, h].T if S0 is not None else np.zeros((dv, dk))
        Amat = [np.exp(g[0, t, h]) * (I - beta[0, t, h] * np.outer(k[0, t, hq], k[0, t, hq])) for t in range(T)]
        for t in range(T):
            prod = I.copy()
            for s in range(t + 1):
                prod = prod @ Amat[s]
            S = S_init @ prod
            for s in range(t + 1):
                tail = I.copy()
                for r in range(s + 1, t + 1):
                    tail = tail @ Amat[r]
                S = S + beta[0, s, h] * np.outer(v[0, s, h], k[0, s, hq]) @ tail
            o[0, t, h] = S @ (scale * q[0, t, hq])
            if t == T - 1:
                final[0, h] = S.T
        if T == 0:
            final[0, h] = S_init.T
    return o, final

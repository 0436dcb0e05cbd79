/*
 * gdn.h - C ABI of the MI355X (gfx950) Gated DeltaNet (GDN) token mixer.
 *
 * The operation is the gated delta rule that the podcast transcript on
 * "On the Design of Qwen3.8-Next Architecture" describes in cue 14: per token,
 * a decay alpha shrinks the whole per-head state, the rule reads what the state
 * holds under the current key, and writes back only the error between the new
 * value and that reading, scaled by a write strength beta.  Cue 4 of the same
 * transcript: the state has a fixed size per head and the cost is linear in the
 * sequence length.  For one head, in math layout (S is dv x dk):
 *
 *     S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *     o_t = S_t (scale * q_t).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - States are stored transposed, M = S^T, as fp32 [N, Hv, dk, dv] row-major:
 *    element (n, h, i, j) = S_{n,h}[j][i], i over the key dim, j over the value dim.
 *  - g is log(alpha) (fp32, <= 0 for a decaying gate); beta is the write strength
 *    after any sigmoid (fp32).  Both are per value head.  g = -inf (alpha = 0, a
 *    full forget) is accepted: the chunked calls floor g at -200 before their
 *    in-chunk prefix sums, where exp(-200) already rounds to 0 in fp32, so the
 *    history before such a token is erased as for alpha = 0 (and the backward's
 *    gradient with respect to such a g is that of g = -200: zero up to rounding).
 *    NaN or +inf gates are not valid input.
 *  - Value head h reads query/key head h / (Hv / Hqk)  (Hv must be a multiple of Hqk).
 *  - q, k, v, o are dtype (fp32 or bf16, see gdn_dtype_t); o is rounded from fp32
 *    accumulators to nearest even.  All tensors are dense, row-major and contiguous.
 *  - Every pointer except `d` is a DEVICE pointer owned by the caller.  The library
 *    allocates no device memory, keeps no mutable global state and may be called
 *    concurrently from several host threads on different streams (except
 *    gdn_fwd_chunked_noalloc, whose static array is shared: see there).
 *  - Work is enqueued asynchronously on `stream` (0 = the null stream); buffers must
 *    stay alive until the stream has passed the work.
 *  - Errors: every call returns a status and never throws, aborts or prints.  All
 *    host-visible arguments are validated before any HIP call.  A failed launch
 *    returns GDN_STATUS_HIP_ERROR; faults inside kernels surface at the caller's
 *    next synchronisation.
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GDN_STATUS_SUCCESS = 0,
  GDN_STATUS_INVALID_VALUE = 1,          /* null required pointer, bad dimension, bad combination */
  GDN_STATUS_NOT_SUPPORTED = 2,          /* valid but not built: head dims, chunk size, dtype */
  GDN_STATUS_MISALIGNED = 3,             /* a pointer is not aligned as documented */
  GDN_STATUS_WORKSPACE_TOO_SMALL = 4,    /* workspace_bytes < gdn_fwd_chunked_workspace_size() */
  GDN_STATUS_HIP_ERROR = 5               /* a HIP runtime call or kernel launch failed */
} gdn_status_t;

typedef enum { GDN_DTYPE_FLOAT32 = 0, GDN_DTYPE_BFLOAT16 = 1 } gdn_dtype_t;

typedef struct {
  int32_t batch;        /* B: batch rows of q/k/v/o; must be 1 when cu_seqlens is given   */
  int32_t seqlen;       /* T: tokens per row (total packed tokens with cu_seqlens); >= 0; */
                        /* B * T >= 2^31 - 256 returns NOT_SUPPORTED (32-bit indices)     */
  int32_t num_seqs;     /* N: number of sequences = B, or len(cu_seqlens) - 1             */
  int32_t num_qk_heads; /* Hqk >= 1                                                       */
  int32_t num_v_heads;  /* Hv >= 1, a multiple of Hqk; NOT_SUPPORTED above 4096          */
  int32_t head_dim_k;   /* dk: 64 or 128                                                  */
  int32_t head_dim_v;   /* dv: 64 or 128 (prefill: dv == dk)                              */
  int32_t chunk_size;   /* prefill chunk length C; 64 is the one built                    */
  float scale;          /* multiplies q; 1.0 gives o_t = S_t q_t                          */
  gdn_dtype_t dtype;    /* element type of q, k, v, o                                     */
} gdn_dims_t;

/*
 * Bytes of device workspace gdn_fwd_chunked needs for these dims (0 when none).
 * Returns 0 as well for dims that gdn_fwd_chunked would reject.
 *
 * Packed sequences (batch 1, 2 <= num_seqs <= 4096) need 4 * num_seqs bytes
 * (rounded up to 256): the sequences are ranked by length on the device and
 * their workgroups numbered longest first, which shortens the launch's tail
 * when lengths are uneven.  The order changes no arithmetic.
 *
 * Otherwise only a row that is long for its number of heads needs one: bf16,
 * dk = dv = 128, no cu_seqlens, B * Hv <= 51 and T >= 3072.  Such a row is cut into S
 * segments run side by side, which relies on the recurrence being affine in the
 * state: the state leaving a segment is Phi M + F, where M is the state
 * entering it, F the state the segment leaves when started from zero and Phi
 * the product of its tokens' transitions exp(g_t) (I - beta_t k_t k_t^T), and
 * each output is its zero-start value plus (scale Phi_t^T q_t)^T M, Phi_t the
 * product up to token t.  The workspace holds scale Phi_t^T q_t per token and
 * value head in bf16 (B * T * Hv * dk * 2 bytes) plus a few fp32 states per
 * segment and value head: 562 MB at B = 1, T = 65536, Hv = 32.
 */
size_t gdn_fwd_chunked_workspace_size(const gdn_dims_t* d);

/*
 * Chunked-parallel prefill: runs the recurrence above over every sequence.
 *
 * The sequence is cut into chunks of C tokens (restarting at every sequence
 * start; the last chunk may be short).  Per chunk and value head, with M the
 * state entering the chunk and G the inclusive in-chunk cumulative sum of g,
 * the chunk is applied as the UT/WY form of the same recurrence:
 *   A = strict_lower(diag(beta) (exp(G_i - G_j) * K K^T)),  T = (I + A)^-1,
 *   W = T diag(beta exp G) K,  U = T diag(beta) V - W M,
 *   O = scale (diag(exp G) Q M + lower_incl_diag(exp(G_i - G_j) * Q K^T) U),
 *   M <- exp(G_C) M + (diag(exp(G_C - G)) K)^T U.
 *
 *   q, k           [B, T, Hqk, dk]  dtype, 16-byte aligned
 *   v              [B, T, Hv, dv]   dtype, 16-byte aligned
 *   g, beta        [B, T, Hv]       fp32, 4-byte aligned
 *   initial_state  [N, Hv, dk, dv]  fp32, 16-byte aligned, or NULL for zeros
 *   cu_seqlens     [N + 1] int32 on the device, or NULL.  With it B must be 1 and
 *                  sequence n is tokens [cu[n], cu[n+1]).  Its contents are the
 *                  caller's contract and are not checked: cu[0] = 0, non-decreasing,
 *                  cu[N] = T.  Empty sequences are allowed (final = initial).
 *   o              [B, T, Hv, dv]   dtype, 16-byte aligned; every token is written
 *   final_state    [N, Hv, dk, dv]  fp32, 16-byte aligned, or NULL (not written).
 *                  It may be the same buffer as initial_state (in-place update);
 *                  any other overlap of an output with an input is undefined.
 *   workspace      device buffer of at least gdn_fwd_chunked_workspace_size(d)
 *                  bytes, 256-byte aligned (may be NULL when that size is 0).
 * Supported: dk = dv in {64, 128}, C = 64, dtype fp32 or bf16.
 */
gdn_status_t gdn_fwd_chunked(const gdn_dims_t* d, const void* q, const void* k, const void* v,
                             const float* g, const float* beta, const float* initial_state,
                             const int32_t* cu_seqlens, void* o, float* final_state,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * gdn_fwd_chunked for callers that cannot allocate: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  Same arguments, layouts
 * and results as gdn_fwd_chunked, without the workspace; it calls no hipMalloc,
 * hipFree or allocating library routine.
 *   - Packed sequences get their longest-first order in a 16 KiB static device
 *     array of the library (one copy per GPU, held until the process ends), so
 *     cu_seqlens may describe at most 4096 sequences: more return
 *     GDN_STATUS_WORKSPACE_TOO_SMALL before any HIP call.
 *   - Rows that gdn_fwd_chunked would cut into segments (bf16, dk = dv = 128,
 *     B * Hv <= 51, T >= 3072) run in one pass of the fused kernel instead: the
 *     same recurrence, different rounding order, slower on such rows.
 *   - Calls that overlap on one GPU (other streams, other threads) share the
 *     static array and race: serialise them.
 *   - The first call on a device looks up that device's copy of the array with
 *     the calling thread's current device, which must be the device of stream
 *     and of the buffers.
 */
gdn_status_t gdn_fwd_chunked_noalloc(const gdn_dims_t* d, const void* q, const void* k, const void* v,
                                     const float* g, const float* beta, const float* initial_state,
                                     const int32_t* cu_seqlens, void* o, float* final_state,
                                     hipStream_t stream);

/*
 * Single-token recurrent decode step for N independent sequences, updating the
 * state in place.  Per (sequence, value head), in stored layout:
 *   r = M^T k,  p = M^T q,  u = beta (v - alpha r),
 *   o = scale (alpha p + (k . q) u),  M <- alpha M + k u^T,
 * which is exactly one step of the recurrence above, with o read after the write.
 *
 *   d->num_seqs = N, d->batch must equal N, d->seqlen must be 1; chunk_size is ignored.
 *   q, k   [N, Hqk, dk]       dtype, 16-byte aligned
 *   v      [N, Hv, dv]        dtype, 16-byte aligned
 *   g, beta [N, Hv]           fp32
 *   state  [N, Hv, dk, dv]    fp32, 16-byte aligned, read and written in place
 *   o      [N, Hv, dv]        dtype, 16-byte aligned
 * Supported: dk, dv in {64, 128}, dtype fp32 or bf16.
 */
gdn_status_t gdn_decode_step(const gdn_dims_t* d, const void* q, const void* k, const void* v,
                             const float* g, const float* beta, float* state, void* o,
                             hipStream_t stream);

/*
 * Multi-token verify from a live state, for speculative decoding: the archdiff
 * model page "Qwen3.8-2.4T-A95B" (components list) drafts tokens with
 * multi-token-prediction modules and verifies them in the target model.  Runs
 * Tv consecutive steps of the recurrence above per sequence, each exactly the
 * step of gdn_decode_step, starting from state_in, in one pass over the state.
 *
 *   d->num_seqs = N, d->batch must equal N, d->seqlen = Tv (1..8; NOT_SUPPORTED
 *   above 8); chunk_size is ignored.
 *   q, k          [N, Tv, Hqk, dk]      dtype, 16-byte aligned
 *   v             [N, Tv, Hv, dv]       dtype, 16-byte aligned
 *   g, beta       [N, Tv, Hv]           fp32
 *   state_in      [N, Hv, dk, dv]       fp32, 16-byte aligned, read
 *   state_out     [N, Hv, dk, dv]       fp32, 16-byte aligned: the state after all Tv
 *                                       tokens, or NULL (not written); may be state_in
 *   token_states  [N, Tv, Hv, dk, dv]   fp32, 16-byte aligned: the state after each
 *                                       token, or NULL.  A caller that accepts the first
 *                                       a tokens continues from token_states[:, a - 1].
 *   o             [N, Tv, Hv, dv]       dtype, 16-byte aligned; o[:, t] reads the state
 *                                       after token t
 * Any overlap of outputs with inputs other than state_out == state_in is undefined.
 * Supported: dk, dv in {64, 128}, dtype fp32 or bf16.
 */
gdn_status_t gdn_decode_verify(const gdn_dims_t* d, const void* q, const void* k, const void* v,
                               const float* g, const float* beta, const float* state_in,
                               float* state_out, float* token_states, void* o, hipStream_t stream);

/*
 * Output epilogue around the mixer: the podcast transcript on "On the Design
 * of Qwen3.8-Next Architecture" (cue 14) adds a sigmoid output gate and a
 * zero-centred RMSNorm to the gated delta rule, and the archdiff model page
 * "Qwen3.8-2.4T-A95B" (components list) writes the gate as sigmoid(x W_g) o.
 * For every row r (one token of one value head, dv values):
 *   y[r] = sigmoid(z[r]) * (o[r] / sqrt(mean_j o[r, j]^2 + eps)) * (1 + weight)
 * with z the gate pre-activations (x W_g, computed by the caller) and weight
 * the zero-centred per-channel norm weight (the scale is 1 + weight).  All in
 * fp32; the sigmoid is 1 / (1 + 2^(-z log2 e)) from the GPU's base-2 exponential
 * and reciprocal, each within about one fp32 ulp.
 *
 *   rows     number of rows, e.g. B * T * Hv for a prefill output; >= 0
 *   dv       values per row: 64 or 128 (NOT_SUPPORTED otherwise)
 *   eps      >= 0
 *   dtype    element type of o, z and y (fp32 or bf16); y is rounded to nearest even
 *   o, z, y  [rows, dv], 16-byte aligned device buffers; y may be o (in place)
 *   weight   [dv] fp32, 16-byte aligned device buffer
 */
gdn_status_t gdn_output_norm_gate(int64_t rows, int32_t dv, float eps, gdn_dtype_t dtype, const void* o,
                                  const void* z, const float* weight, void* y, hipStream_t stream);

/*
 * Pre-mixer step: short causal convolution along the tokens, per channel, and
 * optionally an L2 normalisation of every head.  [Transcript] cue 14 of the
 * podcast on "On the Design of Qwen3.8-Next Architecture" lists short causal
 * convolutions around the rule without a width: the width built here is
 * GDN_SHORT_CONV_WIDTH = 4.  For channel c of token t of a sequence starting
 * at token s (tokens before s count as zero):
 *   y[t, c] = sum_{i < 4} weight[c, i] * x[t - 3 + i, c]
 * and with l2norm != 0 every (token, head) row of head_dim channels is then
 * divided by sqrt(sum of its squares + eps): the per-head q/k normalisation of
 * the archdiff model page "Qwen3.8-2.4T-A95B" (QK-Norm), to unit L2 norm, the
 * scale at which a write with beta = 1 replaces what is stored under a key.
 *
 *   batch, seqlen      B rows of T tokens (with cu_seqlens: B = 1, T = total tokens)
 *   num_seqs           N = B, or len(cu_seqlens) - 1
 *   cu_seqlens         [N + 1] int32 on the device, or NULL (the batch rows are the
 *                      sequences); same contract as for gdn_fwd_chunked
 *   heads, head_dim    channels per token = heads * head_dim; head_dim 64 or 128
 *   eps                >= 0
 *   dtype              element type of x and y (fp32 or bf16); y rounded to nearest even
 *   x, y               [B, T, heads, head_dim], 16-byte aligned; y must not overlap x
 *   weight             [heads * head_dim, 4] fp32, 16-byte aligned (tap i multiplies
 *                      token t - 3 + i)
 */
#define GDN_SHORT_CONV_WIDTH 4
gdn_status_t gdn_short_conv(int32_t batch, int32_t seqlen, int32_t num_seqs, const int32_t* cu_seqlens,
                            int32_t heads, int32_t head_dim, int32_t l2norm, float eps, gdn_dtype_t dtype,
                            const void* x, const float* weight, void* y, hipStream_t stream);

/*
 * Bytes of device workspace gdn_bwd_chunked needs for these dims, each part
 * rounded up to 256 bytes: (N + 1) int32 chunk offsets; two states (dk x dv)
 * per value head and chunk, the state entering the chunk and the gradient of
 * the state leaving it, for (floor(B * T / 64) + N) chunks (a bound on the
 * chunks of any split of the tokens into N sequences); and two values per
 * token, value head and value channel (the chunk form's corrected values U and
 * their gradient).  Values are stored in dtype (bf16 inputs: bf16, the
 * precision in which the matrix cores consume them).  0 for dims with
 * negative sizes.
 */
size_t gdn_bwd_chunked_workspace_size(const gdn_dims_t* d);

/*
 * Backward pass of gdn_fwd_chunked: the gradients of a scalar loss L with
 * respect to q, k, v, g, beta and the initial state, given dL/do for every
 * output token and dL/d(final state).  The report on "On the Design of
 * Qwen3.8-Next Architecture" (paper page, Abstract) weighs every change on
 * training cost as well as inference; the recurrence differentiated is the
 * one at the top of this file (podcast transcript, cue 14), token by token.
 * The result is the exact derivative of that recurrence (up to fp32
 * rounding), whatever chunk form a forward pass used: per token, in stored
 * layout, with alpha = exp(g), Mt = alpha M, r = Mt^T k, u = beta (v - r),
 * M' = Mt + k u^T and o = scale M'^T q, walking the tokens in reverse with dM
 * the gradient of the state after the token:
 *   dM += scale q do^T,  dq = scale M' do,  du = dM^T k,  dv = beta du,
 *   dbeta = du . (v - r),  dr = -beta du,  dk = dM u + Mt dr,
 *   dMt = dM + k dr^T,  dg = <dMt, Mt>,  dM <- alpha dMt.
 * The work runs chunk by chunk on the matrix cores: a forward pass stores each
 * chunk's starting state and U in the workspace, a reverse pass over the chunks
 * carries dM (and stores it per chunk with dZ = (I + A)^-T dU), and a final
 * pass forms every token's gradients, all chunks at once.
 *
 *   d, q, k, v, g, beta, initial_state, cu_seqlens: as for gdn_fwd_chunked
 *                  (the same inputs as the forward pass being differentiated)
 *   d_o            [B, T, Hv, dv]   dtype, 16-byte aligned: dL/do
 *   d_final_state  [N, Hv, dk, dv]  fp32, 16-byte aligned, or NULL for zeros
 *   dq, dk         [B, T, Hqk, dk]  fp32, 16-byte aligned; summed over the value
 *                                   heads that share a query/key head
 *   dv             [B, T, Hv, dv]   fp32, 16-byte aligned
 *   dg, dbeta      [B, T, Hv]       fp32, 4-byte aligned
 *   d_initial_state [N, Hv, dk, dv] fp32, 16-byte aligned, or NULL (not written)
 *   workspace      at least gdn_bwd_chunked_workspace_size(d) bytes, 256-byte
 *                  aligned; its contents on entry and exit are unspecified
 * Every gradient element is written once, with a plain store (no atomics, no
 * clearing pass), and every sum is taken in a fixed order: the same inputs give
 * bitwise the same gradients on every call.  dq and dk are summed over the value
 * heads of a query/key head in one workgroup.  Outputs must not overlap each
 * other or any input.
 * Supported: dk = dv in {64, 128}, C = 64, dtype bf16; dtype fp32 with dk = 64.
 */
gdn_status_t gdn_bwd_chunked(const gdn_dims_t* d, const void* q, const void* k, const void* v,
                             const float* g, const float* beta, const float* initial_state,
                             const int32_t* cu_seqlens, const void* d_o, const float* d_final_state,
                             float* dq, float* dk, float* dv, float* dg, float* dbeta,
                             float* d_initial_state, void* workspace, size_t workspace_bytes,
                             hipStream_t stream);

/* Static, human-readable name of a status code (never NULL). */
const char* gdn_status_string(gdn_status_t s);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H_ */

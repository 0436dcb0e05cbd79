// C ABI of libgdn: argument validation and dispatch to the gfx950 launchers.
// Every host-visible argument is checked before the first HIP call, so invalid
// calls never touch the device.  Nothing here allocates, logs or keeps state.
#include "gdn.h"

#include <stdint.h>
#include <string.h>

#include "launch.hpp"

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool head_dim_ok(int d) { return d == 64 || d == 128; }

// Token indices are 32-bit inside the kernels, which also form a sequence's end plus a chunk length.
constexpr int64_t kMaxTokens = (int64_t(1) << 31) - 256;

// A dtype as the integer the caller stored: a C caller may store any int in a gdn_dtype_t, and reading
// an out-of-range value through the enum type would be undefined in C++.
static_assert(sizeof(gdn_dtype_t) == sizeof(int), "gdn_dtype_t is an int-sized C enum");
int raw_dtype(const gdn_dtype_t& t) {
  int v;
  memcpy(&v, &t, sizeof v);
  return v;
}
bool dtype_ok(const gdn_dtype_t& t) { return raw_dtype(t) == GDN_DTYPE_FLOAT32 || raw_dtype(t) == GDN_DTYPE_BFLOAT16; }
bool is_bf16(const gdn_dtype_t& t) { return raw_dtype(t) == GDN_DTYPE_BFLOAT16; }

// Checks shared by every entry point.
gdn_status_t check_common(const gdn_dims_t* d) {
  if (!d) return GDN_STATUS_INVALID_VALUE;
  if (d->num_qk_heads < 1 || d->num_v_heads < 1 || d->head_dim_k < 1 || d->head_dim_v < 1 || d->num_seqs < 0)
    return GDN_STATUS_INVALID_VALUE;
  if (d->num_v_heads % d->num_qk_heads != 0) return GDN_STATUS_INVALID_VALUE;
  if (!dtype_ok(d->dtype)) return GDN_STATUS_INVALID_VALUE;
  if (!head_dim_ok(d->head_dim_k) || !head_dim_ok(d->head_dim_v)) return GDN_STATUS_NOT_SUPPORTED;
  // The kernels address one token row of q, k, v with 32-bit byte offsets.
  if (d->num_v_heads > 4096) return GDN_STATUS_NOT_SUPPORTED;
  return GDN_STATUS_SUCCESS;
}

gdn_status_t from_hip(hipError_t e) { return e == hipSuccess ? GDN_STATUS_SUCCESS : GDN_STATUS_HIP_ERROR; }

}  // namespace

extern "C" {

size_t gdn_fwd_chunked_workspace_size(const gdn_dims_t* d) {
  // The fused prefill keeps every intermediate in LDS and registers.  Packed
  // sequences (cu_seqlens, so batch 1 and num_seqs > 1) take a few bytes for
  // their longest-first order; a few long bf16 rows (dk = dv = 128, no
  // cu_seqlens) run as segments side by side, with a workspace for the
  // segments' transitions and corrections.
  if (!d || d->batch < 1 || d->seqlen < 0 || d->num_v_heads < 1 || d->chunk_size != 64) return 0;
  if (d->num_seqs != d->batch) return d->batch == 1 ? gdn::order_workspace_bytes(d->num_seqs) : 0;
  if (d->seqlen < 1) return 0;
  if (!is_bf16(d->dtype) || d->head_dim_k != 128 || d->head_dim_v != 128 || d->chunk_size != 64)
    return 0;
  return gdn::seg_workspace_bytes(d->batch, d->seqlen, d->num_v_heads);
}

}  // extern "C"

namespace {

// Checks of a prefill call shared by gdn_fwd_chunked and gdn_fwd_chunked_noalloc (everything but the
// workspace), then its launcher arguments.
gdn_status_t check_fwd(const gdn_dims_t* d, const void* q, const void* k, const void* v, const float* g,
                       const float* beta, const float* initial_state, const int32_t* cu_seqlens, const void* o,
                       const float* final_state) {
  gdn_status_t st = check_common(d);
  if (st != GDN_STATUS_SUCCESS) return st;
  if (d->batch < 0 || d->seqlen < 0) return GDN_STATUS_INVALID_VALUE;
  if (cu_seqlens) {
    if (d->batch != 1) return GDN_STATUS_INVALID_VALUE;
  } else if (d->num_seqs != d->batch) {
    return GDN_STATUS_INVALID_VALUE;
  }
  if (d->chunk_size != 64) return GDN_STATUS_NOT_SUPPORTED;
  if (d->head_dim_k != d->head_dim_v) return GDN_STATUS_NOT_SUPPORTED;
  if (!is_bf16(d->dtype) && d->head_dim_k != 64) return GDN_STATUS_NOT_SUPPORTED;
  const bool has_tokens = static_cast<int64_t>(d->batch) * d->seqlen > 0;
  if (has_tokens && (!q || !k || !v || !g || !beta || !o)) return GDN_STATUS_INVALID_VALUE;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(g, 4) ||
      !aligned(beta, 4) || !aligned(initial_state, 16) || !aligned(final_state, 16) || !aligned(cu_seqlens, 4))
    return GDN_STATUS_MISALIGNED;
  if (static_cast<int64_t>(d->batch) * d->seqlen >= kMaxTokens) return GDN_STATUS_NOT_SUPPORTED;
  return GDN_STATUS_SUCCESS;
}

gdn::PrefillArgs fwd_args(const gdn_dims_t* d, const void* q, const void* k, const void* v, const float* g,
                          const float* beta, const float* initial_state, const int32_t* cu_seqlens, void* o,
                          float* final_state) {
  gdn::PrefillArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = g;
  a.beta = beta;
  a.initial_state = initial_state;
  // One packed sequence is, by the cu_seqlens contract (cu = {0, T}), the single batch row: it takes
  // the batch-row path, which is what gdn_fwd_chunked_workspace_size sized the workspace for.
  a.cu_seqlens = d->num_seqs == 1 ? nullptr : cu_seqlens;
  a.o = o;
  a.final_state = final_state;
  a.batch = d->batch;
  a.seqlen = d->seqlen;
  a.num_seqs = d->num_seqs;
  a.Hqk = d->num_qk_heads;
  a.Hv = d->num_v_heads;
  a.dk = d->head_dim_k;
  a.dv = d->head_dim_v;
  a.chunk = d->chunk_size;
  a.scale = d->scale;
  a.bf16 = is_bf16(d->dtype);
  return a;
}

}  // namespace

extern "C" {

gdn_status_t gdn_fwd_chunked(const gdn_dims_t* d, const void* q, const void* k, const void* v, const float* g,
                             const float* beta, const float* initial_state, const int32_t* cu_seqlens, void* o,
                             float* final_state, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  gdn_status_t st = check_fwd(d, q, k, v, g, beta, initial_state, cu_seqlens, o, final_state);
  if (st != GDN_STATUS_SUCCESS) return st;
  if (!aligned(workspace, 256)) return GDN_STATUS_MISALIGNED;
  const size_t need = gdn_fwd_chunked_workspace_size(d);
  if (workspace_bytes < need) return GDN_STATUS_WORKSPACE_TOO_SMALL;
  if (need > 0 && !workspace) return GDN_STATUS_INVALID_VALUE;
  if (d->num_seqs == 0) return GDN_STATUS_SUCCESS;
  gdn::PrefillArgs a = fwd_args(d, q, k, v, g, beta, initial_state, cu_seqlens, o, final_state);
  a.workspace = workspace;
  a.workspace_bytes = workspace_bytes;
  return from_hip(gdn::launch_prefill(a, stream));
}

gdn_status_t gdn_fwd_chunked_noalloc(const gdn_dims_t* d, const void* q, const void* k, const void* v,
                                     const float* g, const float* beta, const float* initial_state,
                                     const int32_t* cu_seqlens, void* o, float* final_state, hipStream_t stream) {
  gdn_status_t st = check_fwd(d, q, k, v, g, beta, initial_state, cu_seqlens, o, final_state);
  if (st != GDN_STATUS_SUCCESS) return st;
  // The static scratch holds the order of at most kMaxOrderedSeqs packed sequences.
  if (cu_seqlens && d->num_seqs > gdn::kMaxOrderedSeqs) return GDN_STATUS_WORKSPACE_TOO_SMALL;
  if (d->num_seqs == 0) return GDN_STATUS_SUCCESS;
  return from_hip(
      gdn::launch_prefill_noalloc(fwd_args(d, q, k, v, g, beta, initial_state, cu_seqlens, o, final_state), stream));
}

gdn_status_t gdn_decode_step(const gdn_dims_t* d, const void* q, const void* k, const void* v, const float* g,
                             const float* beta, float* state, void* o, hipStream_t stream) {
  gdn_status_t st = check_common(d);
  if (st != GDN_STATUS_SUCCESS) return st;
  if (d->seqlen != 1 || d->batch != d->num_seqs) return GDN_STATUS_INVALID_VALUE;
  if (d->num_seqs == 0) return GDN_STATUS_SUCCESS;
  if (!q || !k || !v || !g || !beta || !state || !o) return GDN_STATUS_INVALID_VALUE;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(state, 16) ||
      !aligned(g, 4) || !aligned(beta, 4))
    return GDN_STATUS_MISALIGNED;
  if (static_cast<int64_t>(d->num_seqs) * d->num_v_heads >= (int64_t(1) << 31)) return GDN_STATUS_NOT_SUPPORTED;

  gdn::DecodeArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = g;
  a.beta = beta;
  a.state = state;
  a.o = o;
  a.num_seqs = d->num_seqs;
  a.Hqk = d->num_qk_heads;
  a.Hv = d->num_v_heads;
  a.dk = d->head_dim_k;
  a.dv = d->head_dim_v;
  a.scale = d->scale;
  a.bf16 = is_bf16(d->dtype);
  return from_hip(gdn::launch_decode(a, stream));
}

gdn_status_t gdn_decode_verify(const gdn_dims_t* d, const void* q, const void* k, const void* v, const float* g,
                               const float* beta, const float* state_in, float* state_out, float* token_states,
                               void* o, hipStream_t stream) {
  gdn_status_t st = check_common(d);
  if (st != GDN_STATUS_SUCCESS) return st;
  if (d->batch != d->num_seqs || d->seqlen < 1) return GDN_STATUS_INVALID_VALUE;
  if (d->seqlen > gdn::kMaxVerifyTokens) return GDN_STATUS_NOT_SUPPORTED;
  if (d->num_seqs == 0) return GDN_STATUS_SUCCESS;
  if (!q || !k || !v || !g || !beta || !state_in || !o) return GDN_STATUS_INVALID_VALUE;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(state_in, 16) ||
      !aligned(state_out, 16) || !aligned(token_states, 16) || !aligned(g, 4) || !aligned(beta, 4))
    return GDN_STATUS_MISALIGNED;
  if (static_cast<int64_t>(d->num_seqs) * d->num_v_heads >= (int64_t(1) << 31)) return GDN_STATUS_NOT_SUPPORTED;

  gdn::VerifyArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = g;
  a.beta = beta;
  a.state_in = state_in;
  a.state_out = state_out;
  a.token_states = token_states;
  a.o = o;
  a.num_seqs = d->num_seqs;
  a.tokens = d->seqlen;
  a.Hqk = d->num_qk_heads;
  a.Hv = d->num_v_heads;
  a.dk = d->head_dim_k;
  a.dv = d->head_dim_v;
  a.scale = d->scale;
  a.bf16 = is_bf16(d->dtype);
  return from_hip(gdn::launch_verify(a, stream));
}

gdn_status_t gdn_output_norm_gate(int64_t rows, int32_t dv, float eps, gdn_dtype_t dtype, const void* o,
                                  const void* z, const float* weight, void* y, hipStream_t stream) {
  if (rows < 0 || dv < 1 || !(eps >= 0.f)) return GDN_STATUS_INVALID_VALUE;
  if (!dtype_ok(dtype)) return GDN_STATUS_INVALID_VALUE;
  if (dv != 64 && dv != 128) return GDN_STATUS_NOT_SUPPORTED;
  if (rows == 0) return GDN_STATUS_SUCCESS;
  if (!o || !z || !weight || !y) return GDN_STATUS_INVALID_VALUE;
  if (!aligned(o, 16) || !aligned(z, 16) || !aligned(y, 16) || !aligned(weight, 16)) return GDN_STATUS_MISALIGNED;
  // 16 threads per row; the grid size must fit in 32 bits.
  if (rows >= (int64_t(1) << 35)) return GDN_STATUS_NOT_SUPPORTED;
  gdn::EpilogueArgs a;
  a.o = o;
  a.z = z;
  a.weight = weight;
  a.y = y;
  a.rows = rows;
  a.dv = dv;
  a.eps = eps;
  a.bf16 = is_bf16(dtype);
  return from_hip(gdn::launch_norm_gate(a, stream));
}

gdn_status_t gdn_short_conv(int32_t batch, int32_t seqlen, int32_t num_seqs, const int32_t* cu_seqlens,
                            int32_t heads, int32_t head_dim, int32_t l2norm, float eps, gdn_dtype_t dtype,
                            const void* x, const float* weight, void* y, hipStream_t stream) {
  if (batch < 0 || seqlen < 0 || num_seqs < 0 || heads < 1 || head_dim < 1 || !(eps >= 0.f))
    return GDN_STATUS_INVALID_VALUE;
  if (!dtype_ok(dtype)) return GDN_STATUS_INVALID_VALUE;
  if (cu_seqlens) {
    if (batch != 1) return GDN_STATUS_INVALID_VALUE;
  } else if (num_seqs != batch) {
    return GDN_STATUS_INVALID_VALUE;
  }
  if (head_dim != 64 && head_dim != 128) return GDN_STATUS_NOT_SUPPORTED;
  const int64_t tokens = static_cast<int64_t>(batch) * seqlen;
  if (tokens == 0 || num_seqs == 0) return GDN_STATUS_SUCCESS;
  if (!x || !weight || !y || x == y) return GDN_STATUS_INVALID_VALUE;
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(weight, 16) || !aligned(cu_seqlens, 4))
    return GDN_STATUS_MISALIGNED;
  // tokens, and runs of 8 tokens times heads, are 32-bit indices in the kernel
  if (tokens >= kMaxTokens || (tokens + 7) / 8 * heads >= (int64_t(1) << 31) - 64)
    return GDN_STATUS_NOT_SUPPORTED;
  gdn::ConvArgs a;
  a.x = x;
  a.weight = weight;
  a.y = y;
  a.cu_seqlens = cu_seqlens;
  a.tokens = static_cast<int>(tokens);
  a.seqlen = seqlen;
  a.num_seqs = num_seqs;
  a.heads = heads;
  a.head_dim = head_dim;
  a.l2norm = l2norm != 0;
  a.eps = eps;
  a.bf16 = is_bf16(dtype);
  return from_hip(gdn::launch_conv(a, stream));
}

size_t gdn_bwd_chunked_workspace_size(const gdn_dims_t* d) {
  if (!d || d->batch < 0 || d->seqlen < 0 || d->num_seqs < 0 || d->num_v_heads < 1 || d->head_dim_k < 1 ||
      d->head_dim_v < 1 || static_cast<int64_t>(d->batch) * d->seqlen >= kMaxTokens)
    return 0;
  return gdn::bwd_parts(static_cast<int64_t>(d->batch) * d->seqlen, d->num_seqs, d->num_v_heads, d->head_dim_k,
                        d->head_dim_v, is_bf16(d->dtype))
      .total;
}

gdn_status_t gdn_bwd_chunked(const gdn_dims_t* d, const void* q, const void* k, const void* v, const float* g,
                             const float* beta, const float* initial_state, const int32_t* cu_seqlens,
                             const void* d_o, const float* d_final_state, float* dq, float* dk, float* dv,
                             float* dg, float* dbeta, float* d_initial_state, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  gdn_status_t st = check_common(d);
  if (st != GDN_STATUS_SUCCESS) return st;
  if (d->batch < 0 || d->seqlen < 0) return GDN_STATUS_INVALID_VALUE;
  if (cu_seqlens) {
    if (d->batch != 1) return GDN_STATUS_INVALID_VALUE;
  } else if (d->num_seqs != d->batch) {
    return GDN_STATUS_INVALID_VALUE;
  }
  if (d->chunk_size != 64) return GDN_STATUS_NOT_SUPPORTED;
  if (d->head_dim_k != d->head_dim_v) return GDN_STATUS_NOT_SUPPORTED;
  if (!is_bf16(d->dtype) && d->head_dim_k != 64) return GDN_STATUS_NOT_SUPPORTED;
  const bool has_tokens = static_cast<int64_t>(d->batch) * d->seqlen > 0;
  if (has_tokens && (!q || !k || !v || !g || !beta || !d_o || !dq || !dk || !dv || !dg || !dbeta))
    return GDN_STATUS_INVALID_VALUE;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(d_o, 16) || !aligned(g, 4) ||
      !aligned(beta, 4) || !aligned(initial_state, 16) || !aligned(d_final_state, 16) ||
      !aligned(cu_seqlens, 4) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) || !aligned(dg, 4) ||
      !aligned(dbeta, 4) || !aligned(d_initial_state, 16) || !aligned(workspace, 256))
    return GDN_STATUS_MISALIGNED;
  if (d->num_seqs == 0) return GDN_STATUS_SUCCESS;
  const size_t need = gdn_bwd_chunked_workspace_size(d);
  if (workspace_bytes < need) return GDN_STATUS_WORKSPACE_TOO_SMALL;
  if (need > 0 && !workspace) return GDN_STATUS_INVALID_VALUE;
  // Token indices are 32-bit inside the kernels, and so is the grid of up to 16 workgroups per unit.
  if (static_cast<int64_t>(d->batch) * d->seqlen >= kMaxTokens ||
      static_cast<int64_t>(d->num_seqs) * d->num_v_heads * 16 >= (int64_t(1) << 31))
    return GDN_STATUS_NOT_SUPPORTED;

  gdn::BwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.dout = d_o;
  a.g = g;
  a.beta = beta;
  a.initial_state = initial_state;
  a.d_final_state = d_final_state;
  a.cu_seqlens = cu_seqlens;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dg = dg;
  a.dbeta = dbeta;
  a.d_initial_state = d_initial_state;
  a.workspace = workspace;
  a.batch = d->batch;
  a.seqlen = d->seqlen;
  a.num_seqs = d->num_seqs;
  a.Hqk = d->num_qk_heads;
  a.Hv = d->num_v_heads;
  a.head_dim_k = d->head_dim_k;
  a.head_dim_v = d->head_dim_v;
  a.scale = d->scale;
  a.bf16 = is_bf16(d->dtype);
  return from_hip(gdn::launch_bwd(a, stream));
}

const char* gdn_status_string(gdn_status_t s) {
  switch (s) {
    case GDN_STATUS_SUCCESS: return "GDN_STATUS_SUCCESS";
    case GDN_STATUS_INVALID_VALUE: return "GDN_STATUS_INVALID_VALUE: invalid argument";
    case GDN_STATUS_NOT_SUPPORTED: return "GDN_STATUS_NOT_SUPPORTED: configuration not built";
    case GDN_STATUS_MISALIGNED: return "GDN_STATUS_MISALIGNED: pointer not aligned";
    case GDN_STATUS_WORKSPACE_TOO_SMALL: return "GDN_STATUS_WORKSPACE_TOO_SMALL";
    case GDN_STATUS_HIP_ERROR: return "GDN_STATUS_HIP_ERROR: HIP call or kernel launch failed";
  }
  return "GDN_STATUS_UNKNOWN";
}

}  // extern "C"

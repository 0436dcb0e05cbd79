// Internal interface between the C ABI (gdn_api.cpp) and the kernel launchers.
// Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

struct DecodeArgs {
  const void *q, *k, *v;
  const float *g, *beta;
  float* state;
  void* o;
  int num_seqs, Hqk, Hv, dk, dv;
  float scale;
  bool bf16;
};

struct PrefillArgs {
  const void *q, *k, *v;
  const float *g, *beta;
  const float* initial_state;  // may be null (zeros)
  const int32_t* cu_seqlens;   // may be null (batch rows are the sequences)
  void* o;
  float* final_state;          // may be null
  int batch, seqlen, num_seqs, Hqk, Hv, dk, dv, chunk;
  float scale;
  bool bf16;
  // Set by the backward pass only: keep every chunk's starting state
  // ([chunk][Hv][dk][dv], chunk = chunk_base[n] + local index) and U (the
  // chunk form's corrected values, [token][Hv][dv]) in the element type of
  // q, k, v, and skip o.
  void* save_state = nullptr;
  void* save_u = nullptr;
  const int32_t* chunk_base = nullptr;  // [N + 1] with cu_seqlens, else null (n * ceil(T / C))
  // Caller's workspace (segmented prefill of long rows, see seg_plan; the
  // longest-first order of packed sequences, see order_workspace_bytes).
  void* workspace = nullptr;
  size_t workspace_bytes = 0;
  // Set by launch_prefill: the sequences in the order their workgroups are
  // numbered ([N] int32 on the device), or null for the natural order.
  const int32_t* order = nullptr;
};

// Workspace bytes for the longest-first order of num_seqs packed sequences
// (0 where the natural order is kept: fewer than 2 or more than kMaxOrderedSeqs).
constexpr int kMaxOrderedSeqs = 4096;
size_t order_workspace_bytes(int num_seqs);

// Segmented prefill of a few long batch rows (bf16, dk = dv = 128, no cu_seqlens):
// every row is cut into nseg segments of seg_len tokens that run side by side.
struct SegPlan {
  int nseg = 0, seg_len = 0;
  void* qt = nullptr;       // [B, T, Hv, dk] bf16: the transition runs' outputs
  float* fin = nullptr;     // [nseg][B][Hv][dk][dv] fp32: end states from the zero state (segment 0: the row's)
  float* phi = nullptr;     // [nseg][B][Hv][dk][dk] fp32: transitions of the segments
  void* mstart = nullptr;   // [nseg][B][Hv][dv][dk] bf16: start states of the segments, transposed
  float* mbuf = nullptr;    // two [B][Hv][dk][dv] fp32 buffers for the scan
  size_t mbuf_stride = 0;   // floats between them
};
// Whether (and how) rows of T tokens are segmented for batch * Hv units.
bool seg_plan(int batch, int T, int Hv, SegPlan* sp);
size_t seg_workspace_bytes(int batch, int T, int Hv);  // 0 when not segmented
void seg_carve(void* ws, int batch, int T, int Hv, SegPlan* sp);
hipError_t launch_seg_finish(const PrefillArgs& a, const SegPlan& sp, hipStream_t stream);

// Multi-token verify: Tv (<= kMaxVerifyTokens) consecutive steps per sequence.
constexpr int kMaxVerifyTokens = 8;

struct VerifyArgs {
  const void *q, *k, *v;
  const float *g, *beta;
  const float* state_in;
  float* state_out;     // may be null (not written) or state_in
  float* token_states;  // may be null
  void* o;
  int num_seqs, tokens, Hqk, Hv, dk, dv;
  float scale;
  bool bf16;
};

// Output epilogue: rows of dv values, y = sigmoid(z) * o / rms(o) * (1 + w).
struct EpilogueArgs {
  const void *o, *z;
  const float* weight;
  void* y;
  int64_t rows;
  int dv;
  float eps;
  bool bf16;
};

// Short causal convolution (width 4) along the tokens, per channel, optionally
// followed by an L2 normalisation of every (token, head) row.
struct ConvArgs {
  const void* x;
  const float* weight;  // [heads * head_dim, 4]
  void* y;
  const int32_t* cu_seqlens;  // may be null: batch rows are the sequences
  int tokens, seqlen, num_seqs, heads, head_dim;
  bool l2norm;
  float eps;
  bool bf16;
};

// Backward pass of a prefill: fp32 gradients of q, k, v, g, beta and the initial state.
struct BwdArgs {
  const void *q, *k, *v, *dout;
  const float *g, *beta;
  const float* initial_state;  // may be null (zeros)
  const float* d_final_state;  // may be null (zeros)
  const int32_t* cu_seqlens;   // may be null
  float *dq, *dk, *dv, *dg, *dbeta;
  float* d_initial_state;      // may be null (not written)
  void* workspace;             // bwd_parts(...).total bytes, 256-byte aligned
  int batch, seqlen, num_seqs, Hqk, Hv, head_dim_k, head_dim_v;
  float scale;
  bool bf16;
};
// Workspace of the backward pass (byte offsets of its parts and the total size).
struct BwdParts {
  size_t cpre = 0, state = 0, dm = 0, u = 0, dz = 0, total = 0;
};
BwdParts bwd_parts(int64_t tokens, int num_seqs, int Hv, int dk, int dv, bool bf16);

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream);
hipError_t launch_conv(const ConvArgs& a, hipStream_t stream);
hipError_t launch_norm_gate(const EpilogueArgs& a, hipStream_t stream);
hipError_t launch_verify(const VerifyArgs& a, hipStream_t stream);
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);
// The prefill without a caller's workspace: the fused kernel for every unit count, and for packed
// sequences (at most kMaxOrderedSeqs) the longest-first order in a static device array of the library.
hipError_t launch_prefill_noalloc(const PrefillArgs& a, hipStream_t stream);

}  // namespace gdn

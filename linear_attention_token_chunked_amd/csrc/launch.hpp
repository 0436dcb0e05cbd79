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
  // Caller's workspace (two-pass prefill of few units, see two_pass_parts; the
  // longest-first order of packed sequences, see order_workspace_bytes).
  void* workspace = nullptr;
  size_t workspace_bytes = 0;
  // Set by launch_prefill: the sequences in the order their workgroups are
  // numbered ([N] int32 on the device), or null for the natural order.
  const int32_t* order = nullptr;
};

// Workspace bytes for the longest-first order of num_seqs packed sequences
// (0 where the natural order is kept: fewer than 2 or more than 4096 sequences).
size_t order_workspace_bytes(int num_seqs);
// Ranks packed sequences by length, longest first (order[rank] = sequence).
hipError_t launch_order(const int32_t* cu, int num_seqs, int32_t* order, hipStream_t stream);

// Two-pass prefill of few (sequence, value head) units (bf16, dk = dv = 128): a
// chunk-parallel pass writes every (chunk, value head)'s T = (I + A)^-1, masked
// Q K^T and gate vectors to the workspace, and a sequential pass per unit runs
// only the recurrence and the outputs from them.
constexpr int kTwoPassBlockBytes = 13312;  // per (chunk slot, value head)
constexpr int kTwoPassMaxUnits = 128;      // (sequence, value head) units up to which it runs
struct TwoPassParts {
  int64_t slots = 0;  // chunk slots: B * ceil(T / 64), or T / 64 + N for packed sequences
  size_t chunk_base = 0, order = 0, blocks = 0, total = 0;  // byte offsets in the workspace; total size
};
bool two_pass_applies(bool bf16, int dk, int dv, int num_seqs, int Hv, int seqlen);
TwoPassParts two_pass_parts(int batch, int T, int N, bool packed, int Hv);
hipError_t launch_two_pass(const PrefillArgs& a, hipStream_t stream);
// Exclusive prefix sum of the packed sequences' chunk counts (ceil(L_n / 64)): chunk_base[n] is
// sequence n's first chunk slot, chunk_base[N] the number of slots.
hipError_t launch_chunk_base(const int32_t* cu, int num_seqs, int32_t* chunk_base, hipStream_t stream);

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
  void* workspace;             // bwd_workspace_bytes, 256-byte aligned
  int batch, seqlen, num_seqs, Hqk, Hv, head_dim_k, head_dim_v;
  float scale;
  bool bf16;
};
struct BwdParts {
  size_t cpre = 0, state = 0, dm = 0, u = 0, dz = 0, total = 0;  // byte offsets in the workspace; total size
};
BwdParts bwd_parts(int64_t tokens, int num_seqs, int Hv, int dk, int dv, bool bf16);

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream);
hipError_t launch_conv(const ConvArgs& a, hipStream_t stream);
hipError_t launch_norm_gate(const EpilogueArgs& a, hipStream_t stream);
hipError_t launch_verify(const VerifyArgs& a, hipStream_t stream);
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);

}  // namespace gdn

// Host-side planning shared by the C ABI and the launchers: which prefill path a
// call takes and how the caller's workspace is laid out.  Plain C++ with no
// device code, so that the argument checking of the C ABI can also be built and
// exercised on the host alone (with the sanitizers) together with it.
#include <stddef.h>
#include <stdint.h>

#include "launch.hpp"

namespace gdn {
namespace {

constexpr int C = 64;           // chunk length
constexpr int kMaxOrdered = 4096;  // beyond this many packed sequences the natural order is kept
size_t al256(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace

size_t order_workspace_bytes(int num_seqs) {
  return num_seqs >= 2 && num_seqs <= kMaxOrdered ? al256(static_cast<size_t>(num_seqs) * 4) : 0;
}

bool two_pass_applies(bool bf16, int dk, int dv, int num_seqs, int Hv, int seqlen) {
  const int64_t units = static_cast<int64_t>(num_seqs) * Hv;
  return bf16 && dk == 128 && dv == 128 && units >= 1 && units <= kTwoPassMaxUnits && seqlen >= 1;
}

// Workspace of the two-pass prefill: [chunk_base: N + 1 int32 (packed only)] [order: N int32 (packed,
// 2 <= N <= 4096)] [blocks: slots x Hv x kTwoPassBlockBytes], each part 256-byte aligned.  Packed
// sequences need at most T / 64 + N chunk slots (every sequence's partial last chunk adds one).
TwoPassParts two_pass_parts(int batch, int T, int N, bool packed, int Hv) {
  TwoPassParts w;
  w.slots = packed ? static_cast<int64_t>(T) / C + N : static_cast<int64_t>(batch) * ((T + C - 1) / C);
  w.chunk_base = 0;
  w.order = packed ? al256(static_cast<size_t>(N + 1) * 4) : 0;
  w.blocks = w.order + (packed ? order_workspace_bytes(N) : 0);
  w.total = w.blocks + static_cast<size_t>(w.slots) * Hv * kTwoPassBlockBytes;
  return w;
}

// Workspace of the backward pass: [N + 1 int32 chunk offsets] and, in the input dtype, the state
// entering every chunk and the state gradient per chunk ((T / 64 + N) chunks x Hv x dk x dv), then U
// and dZ per token (tokens x Hv x dv); each part 256-byte aligned.
BwdParts bwd_parts(int64_t tokens, int num_seqs, int Hv, int dk, int dv, bool bf16) {
  const size_t esize = bf16 ? 2 : 4;
  const size_t chunks = static_cast<size_t>(tokens / C + num_seqs);
  BwdParts w;
  w.cpre = 0;
  w.state = al256(static_cast<size_t>(num_seqs + 1) * 4);
  w.dm = w.state + al256(chunks * Hv * dk * dv * esize);
  w.u = w.dm + al256(chunks * Hv * dk * dv * esize);
  w.dz = w.u + al256(static_cast<size_t>(tokens) * Hv * dv * esize);
  w.total = w.dz + al256(static_cast<size_t>(tokens) * Hv * dv * esize);
  return w;
}

}  // namespace gdn

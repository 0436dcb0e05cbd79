// Host-side planning shared by the C ABI and the launchers: how the callers'
// workspaces are laid out and which prefill path a call takes.  Plain C++ with
// no device code, so that the argument checking of the C ABI can be built for
// the host alone, with the sanitizers, together with the real sizing logic.
#include <stddef.h>
#include <stdint.h>

#include <algorithm>

#include "launch.hpp"

namespace gdn {
namespace {

constexpr int64_t C = 64;              // chunk length
constexpr int64_t D = 128;             // dk = dv of the segmented prefill
constexpr int64_t kComputeUnits = 256;  // gfx950 compute units one launch fills

size_t al256(size_t x) { return (x + 255) / 256 * 256; }

// Byte offsets of the segmented prefill's workspace parts (the layout seg_carve hands out).
struct SegParts {
  size_t qt, fin, phi, mstart, mbuf, total;
};
SegParts seg_parts(int batch, int T, int Hv, int nseg) {
  const size_t mat = static_cast<size_t>(D) * D;
  SegParts w;
  w.qt = 0;                                                                       // [B, T, Hv, dk] bf16
  w.fin = al256(static_cast<size_t>(batch) * T * Hv * D * 2);                     // [nseg, B, Hv, dk, dv] fp32
  w.phi = w.fin + al256(static_cast<size_t>(nseg) * batch * Hv * mat * 4);        // [nseg, B, Hv, dk, dk] fp32
  w.mstart = w.phi + al256(static_cast<size_t>(nseg) * batch * Hv * mat * 4);     // [nseg, B, Hv, dv, dk] bf16
  w.mbuf = w.mstart + al256(static_cast<size_t>(nseg) * batch * Hv * mat * 2);    // 2 x [B, Hv, dk, dv] fp32
  w.total = w.mbuf + 2 * al256(static_cast<size_t>(batch) * Hv * mat * 4);
  return w;
}

}  // namespace

size_t order_workspace_bytes(int num_seqs) {
  return num_seqs >= 2 && num_seqs <= kMaxOrderedSeqs ? al256(static_cast<size_t>(num_seqs) * 4) : 0;
}

bool seg_plan(int batch, int T, int Hv, SegPlan* sp) {
  const int64_t units = static_cast<int64_t>(batch) * Hv;
  if (units <= 0 || units > kComputeUnits || T <= 0) return false;
  // 2 nseg - 1 runs per unit fill at most every compute unit (one 128-column
  // workgroup each), each segment holds at least 16 chunks, and fewer than
  // three segments would not pay for the wider slices and the extra runs
  int64_t nseg = std::min((kComputeUnits / units + 1) / 2, static_cast<int64_t>(T) / (16 * C));
  if (nseg < 3) return false;
  const int64_t nch = (static_cast<int64_t>(T) + C - 1) / C;
  const int64_t len = (nch + nseg - 1) / nseg * C;
  nseg = (static_cast<int64_t>(T) + len - 1) / len;  // (no empty segment)
  if (nseg < 3) return false;
  sp->nseg = static_cast<int>(nseg);
  sp->seg_len = static_cast<int>(len);
  return true;
}

size_t seg_workspace_bytes(int batch, int T, int Hv) {
  SegPlan sp;
  if (!seg_plan(batch, T, Hv, &sp)) return 0;
  return seg_parts(batch, T, Hv, sp.nseg).total;
}

void seg_carve(void* ws, int batch, int T, int Hv, SegPlan* sp) {
  const SegParts w = seg_parts(batch, T, Hv, sp->nseg);
  unsigned char* base = static_cast<unsigned char*>(ws);
  sp->qt = base + w.qt;
  sp->fin = reinterpret_cast<float*>(base + w.fin);
  sp->phi = reinterpret_cast<float*>(base + w.phi);
  sp->mstart = base + w.mstart;
  sp->mbuf = reinterpret_cast<float*>(base + w.mbuf);
  sp->mbuf_stride = (w.total - w.mbuf) / 2 / sizeof(float);
}

// Workspace of the backward pass: [N + 1 int32 chunk offsets] and, in the input dtype, the state
// entering every chunk and the state gradient per chunk ((tokens / 64 + N) chunks x Hv x dk x dv), then
// U and dZ per token (tokens x Hv x dv); each part 256-byte aligned.
BwdParts bwd_parts(int64_t tokens, int num_seqs, int Hv, int dk, int dv, bool bf16) {
  const size_t esize = bf16 ? 2 : 4;
  const size_t chunks = static_cast<size_t>(tokens / C + num_seqs);
  BwdParts w;
  w.cpre = 0;
  w.state = al256((static_cast<size_t>(num_seqs) + 1) * 4);
  w.dm = w.state + al256(chunks * Hv * dk * dv * esize);
  w.u = w.dm + al256(chunks * Hv * dk * dv * esize);
  w.dz = w.u + al256(static_cast<size_t>(tokens) * Hv * dv * esize);
  w.total = w.dz + al256(static_cast<size_t>(tokens) * Hv * dv * esize);
  return w;
}

}  // namespace gdn

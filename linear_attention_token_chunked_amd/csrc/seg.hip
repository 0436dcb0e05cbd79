// Segmented prefill of a few long sequences, gfx950.
//
// The recurrence of the podcast transcript on "On the Design of Qwen3.8-Next
// Architecture" (cue 14) is affine in the state: over a run of tokens the state
// leaving the run is Phi M + F, where M is the state entering it, Phi the
// ordered product of the tokens' transitions alpha_t (I - beta_t k_t k_t^T)
// (stored layout) and F the end state of the same run started from zero; and
// every output inside the run is o_t = o_t(0) + (scale Phi_t^T q_t)^T M with
// Phi_t the product up to token t.  A row with few units leaves most compute
// units idle while one workgroup per unit walks all its chunks in order, so the
// row is cut into nseg segments and one launch runs, side by side:
//   segment 0 from the row's initial state (outputs and end state final);
//   every later segment from the zero state (o(0) into o, and F);
//   every later segment with v = 0 from the identity state: its outputs are
//   scale Phi_t^T q_t ("qt"), its end state Phi.
// A scan over the segments then gives each segment's start state,
// M_{s+1} = Phi_s M_s + F_s, and the row's final state; a correction adds
// qt_t^T M_s to every output of segment s >= 1.  The two finishing kernels run
// on the matrix cores (the scan in fp32, the correction with bf16 operands).
#include <algorithm>

#include "device_common.hpp"
#include "launch.hpp"

namespace gdn {
namespace {

constexpr int C = 64;
constexpr int D = 128;  // dk = dv
constexpr int kComputeUnits = 256;

// -------------------------------------------------------------- segment scan
// One step of M_{s+1} = Phi_s M_s + F_s for every (row, value head), in fp32:
// eight workgroups per unit, one 16-row band of the result each.  Each band
// also writes its 16 columns of M_s, transposed and in bf16, as the
// correction's operand.
constexpr int LDS_F = D + 4;  // fp32 rows (16-byte aligned, 4-bank shift per row)

__global__ __launch_bounds__(256) void seg_scan_step_kernel(const float* mcur, const float* phi_s, const float* fin_s,
                                                            float* mnext, bf16* mstart_s) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  float* sM = reinterpret_cast<float*>(smem);  // [D][LDS_F]: M, row-major
  float* sPhi = sM + D * LDS_F;                // [16][LDS_F]: the band's rows of Phi
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lg = lane >> 4, lr = lane & 15;
  const int unit = blockIdx.x >> 3, band = blockIdx.x & 7;
  const size_t mat = static_cast<size_t>(D) * D;
  const float* m = mcur + unit * mat;
  const float* ph = phi_s + unit * mat + static_cast<size_t>(16 * band) * D;
  constexpr int NM = D * D / 4 / 256, NP = 16 * D / 4 / 256;
  floatx4 vm[NM], vp[NP];
#pragma unroll
  for (int it = 0; it < NM; ++it) vm[it] = *reinterpret_cast<const floatx4*>(m + 4 * (tid + 256 * it));
#pragma unroll
  for (int it = 0; it < NP; ++it) vp[it] = *reinterpret_cast<const floatx4*>(ph + 4 * (tid + 256 * it));
#pragma unroll
  for (int it = 0; it < NM; ++it) {
    const int i = tid + 256 * it, r = i / (D / 4), e = (i - r * (D / 4)) * 4;
    *reinterpret_cast<floatx4*>(sM + r * LDS_F + e) = vm[it];
  }
#pragma unroll
  for (int it = 0; it < NP; ++it) {
    const int i = tid + 256 * it, r = i / (D / 4), e = (i - r * (D / 4)) * 4;
    *reinterpret_cast<floatx4*>(sPhi + r * LDS_F + e) = vp[it];
  }
  __syncthreads();
  if (mstart_s) {  // rows 16 band .. 16 band + 15 of M_s^T: 8 consecutive k per thread
    const int j = 16 * band + (tid >> 4), k0 = (tid & 15) * 8;
    bf16x8 w;
#pragma unroll
    for (int u = 0; u < 8; ++u) w[u] = from_float<bf16>(sM[(k0 + u) * LDS_F + j]);
    *reinterpret_cast<bf16x8*>(mstart_s + unit * mat + static_cast<size_t>(j) * D + k0) = w;
  }
  // (Phi M)[i][j] = sum_k Phi[i][k] M[k][j]; wavefront w: column tiles 2w, 2w + 1.
  // In k-group kg lane group g supplies k = 16 kg + 4 g + (0..3) for both operands.
  const float* fs = fin_s + unit * mat;
  float* out = mnext + unit * mat;
#pragma unroll
  for (int jj = 0; jj < 2; ++jj) {
    const int tj = 2 * wave + jj;
    floatx4 acc = zero4();
    const float* ar = sPhi + lr * LDS_F;
#pragma unroll
    for (int kg = 0; kg < D / Mma<float>::KG; ++kg) {
      const float* bc = sM + (16 * kg + 4 * lg) * LDS_F + 16 * tj + lr;
      const floatx4 b = {bc[0], bc[LDS_F], bc[2 * LDS_F], bc[3 * LDS_F]};
      Mma<float>::mma(acc, lds_frag<float>(ar, kg, lane), b);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const size_t at = static_cast<size_t>(16 * band + 4 * lg + r) * D + 16 * tj + lr;
      out[at] = acc[r] + fs[at];
    }
  }
}

// ----------------------------------------------------------------- correction
// o_t += qt_t^T M_s for the tokens of segments s >= 1: one workgroup per
// (row, segment, block of 512 tokens, value head), 64 tokens at a time, the
// output tile staged through LDS so that o is read and written in whole rows.
constexpr int LDS_B = D + 16;  // bf16 rows of 288 bytes
constexpr int kCorrTokens = 512;

__global__ __launch_bounds__(256) void seg_correct_kernel(bf16* o, const bf16* qt, const bf16* mstart, int batch,
                                                          int T, int Hv, int nseg, int seg_len, int nblk) {
  __shared__ __attribute__((aligned(16))) bf16 sMt[D * LDS_B];  // M_s^T rows
  __shared__ __attribute__((aligned(16))) bf16 sQt[C * LDS_B];  // 64 token rows of qt
  __shared__ __attribute__((aligned(16))) bf16 sO[C * LDS_B];   // the same rows of o
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lg = lane >> 4, lr = lane & 15;
  int id = blockIdx.x;
  const int h = id % Hv;
  id /= Hv;
  const int blk = id % nblk;
  id /= nblk;
  const int s = 1 + id % (nseg - 1);
  const int b = id / (nseg - 1);
  const int bos = b * T + s * seg_len, eos = min(b * T + T, bos + seg_len);
  const int t0 = bos + blk * kCorrTokens, t1 = min(eos, t0 + kCorrTokens);
  if (t0 >= t1) return;
  const size_t row = static_cast<size_t>(Hv) * D;  // elements per token of o / qt
  const bf16* ms = mstart + ((static_cast<size_t>(s) * batch + b) * Hv + h) * D * D;
  for (int i = tid; i < D * D / 8; i += 256) {
    const int r = i / (D / 8), e = (i - r * (D / 8)) * 8;
    *reinterpret_cast<bf16x8*>(sMt + r * LDS_B + e) = *reinterpret_cast<const bf16x8*>(ms + r * D + e);
  }
  constexpr int IT = C * D / 8 / 256;
  bf16x8 vq[IT], vo[IT];
  auto fetch = [&](int tt) {  // the tile's rows of qt and o into registers (streaming: read once)
    const int L = min(C, t1 - tt);
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int i = tid + it * 256, r = i / (D / 8), e = (i - r * (D / 8)) * 8;
      vq[it] = bf16x8{};
      vo[it] = bf16x8{};
      if (r < L) {
        const size_t at = (tt + r) * row + h * D + e;
        vq[it] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(qt + at));
        vo[it] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(o + at));
      }
    }
  };
  fetch(t0);
  for (int tt = t0; tt < t1; tt += C) {
    const int L = min(C, t1 - tt);
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int i = tid + it * 256, r = i / (D / 8), e = (i - r * (D / 8)) * 8;
      *reinterpret_cast<bf16x8*>(sQt + r * LDS_B + e) = vq[it];
      *reinterpret_cast<bf16x8*>(sO + r * LDS_B + e) = vo[it];
    }
    lds_barrier();  // (the previous tile's stores to o may still be in flight)
    if (tt + C < t1) fetch(tt + C);  // in flight during this tile's products
    // 4 x 8 output tiles, formed transposed (o^T += M_s^T qt^T) so that a lane holds four adjacent
    // columns of one token row: one 8-byte update per lane and tile; wavefront w owns column tiles
    // 2w and 2w + 1
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int jt = 2 * wave + jj;
      const bf16* ar = sMt + (16 * jt + lr) * LDS_B;
      Mma<bf16>::frag af[D / 32];
#pragma unroll
      for (int kg = 0; kg < D / 32; ++kg) af[kg] = lds_frag<bf16>(ar, kg, lane);
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        floatx4 acc = zero4();
        const bf16* br = sQt + (16 * it + lr) * LDS_B;
#pragma unroll
        for (int kg = 0; kg < D / 32; ++kg) Mma<bf16>::mma(acc, af[kg], lds_frag<bf16>(br, kg, lane));
        // acc[r]: token 16 it + lr, column 16 jt + 4 lg + r (each element has one owner)
        bf16x4* x = reinterpret_cast<bf16x4*>(sO + (16 * it + lr) * LDS_B + 16 * jt + 4 * lg);
        bf16x4 ov = *x;
#pragma unroll
        for (int r = 0; r < 4; ++r) ov[r] = from_float<bf16>(to_float(ov[r]) + acc[r]);
        *x = ov;
      }
    }
    lds_barrier();
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int i = tid + it * 256, r = i / (D / 8), e = (i - r * (D / 8)) * 8;
      if (r < L)
        __builtin_nontemporal_store(*reinterpret_cast<const bf16x8*>(sO + r * LDS_B + e),
                                    reinterpret_cast<bf16x8*>(o + (tt + r) * row + h * D + e));
    }
    lds_barrier();
  }
}

}  // namespace

hipError_t launch_seg_finish(const PrefillArgs& a, const SegPlan& sp, hipStream_t stream) {
  const size_t scan_lds = (D + 16) * LDS_F * sizeof(float);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&seg_scan_step_kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(scan_lds));
  if (e != hipSuccess) return e;
  const size_t block = static_cast<size_t>(a.batch) * a.Hv * D * D;  // one segment's states
  const float* m = sp.fin;  // M_1 = the end of segment 0
  for (int s = 1; s < sp.nseg; ++s) {
    // M_{s+1} into a work buffer, or for the last segment into the final state (when asked for)
    float* next = (s + 1 == sp.nseg && a.final_state) ? a.final_state : sp.mbuf + (s & 1) * sp.mbuf_stride;
    seg_scan_step_kernel<<<dim3(a.batch * a.Hv * 8), dim3(256), scan_lds, stream>>>(
        m, sp.phi + s * block, sp.fin + s * block, next, static_cast<bf16*>(sp.mstart) + s * block);
    m = next;
  }
  const int nblk = (sp.seg_len + kCorrTokens - 1) / kCorrTokens;
  const int64_t groups = static_cast<int64_t>(a.batch) * (sp.nseg - 1) * nblk * a.Hv;
  seg_correct_kernel<<<dim3(static_cast<unsigned>(groups)), dim3(256), 0, stream>>>(
      static_cast<bf16*>(a.o), static_cast<const bf16*>(sp.qt), static_cast<const bf16*>(sp.mstart), a.batch,
      a.seqlen, a.Hv, sp.nseg, sp.seg_len, nblk);
  return hipGetLastError();
}

}  // namespace gdn

// Two-pass chunked prefill for few (sequence, value head) units, bf16, dk = dv = 128.
//
// Method: the recurrence of the podcast transcript on "On the Design of
// Qwen3.8-Next Architecture", cue 14 (decay the whole state, read what the key
// holds, write only the error), in the stored layout M = S^T.  Per chunk of
// C = 64 tokens starting from state M (G the inclusive in-chunk cumsum of g):
//   A = strict_lower(beta_i exp(G_i - G_j) (K K^T)_ij),   T = (I + A)^-1
//   Z = diag(beta) (V - diag(exp G) K M),                  U = T Z
//   O = scale (diag(exp G) Q M + P U),  P = lower_incl(exp(G_i - G_j) (Q K^T)_ij)
//   M <- exp(G_C) M + K^T diag(exp(G_C - G)) U
// (the UT form of the chunk, exact in real arithmetic: U = T diag(beta) V - W M
// with W = T diag(beta exp G) K).
//
// With few units the chip holds far more compute units than recurrences, and
// the time of a launch is the chunk count times the time one workgroup takes
// per chunk.  Everything that does not depend on the state is therefore moved
// out of the sequential loop:
//   prep_kernel   every (chunk, query/key head) at once: the Gram products
//                 K K^T and Q K^T, and per value head the gate scan, A, the
//                 full inverse T (diagonal 16x16 blocks by forward substitution,
//                 the blocks below them with fp32 matrix-core products) and P.
//                 T and P go to the workspace in bf16 matrix-core operand order,
//                 with the chunk's gate vectors.
//   scan_kernel   one workgroup per (unit, 32-column slice of dv) walks the
//                 chunks in order with the fp32 state slice in registers.  Per
//                 chunk its recurrence wavefronts form only K M, Z, U = T Z and
//                 the state update; output wavefronts form O from the state and
//                 U they are handed through LDS; stager wavefronts copy the next
//                 chunk's K, Q, V and its workspace block into LDS.
#include "launch.hpp"
#include "prefill_common.hpp"

namespace gdn {
namespace {

constexpr int D = 128;      // dk = dv
constexpr int KGK = D / 32;  // 32-wide k-groups over the key dim
constexpr int LDK = D + 16;  // padded K / Q rows (bf16 elements; see Layout in prefill.hip)
constexpr int LDF = 68;      // fp32 rows of the prep kernel's 64 x 64 matrices (16-byte aligned, bank shift 4)
constexpr int LDA = 20;      // fp32 rows of the diagonal blocks of A, transposed

// ---------------------------------------------------------------- workspace block of one (chunk, value head)
// T and P as bf16 operand fragments: fragment (ct, kg) holds, for lane (lg, lr), row 16 ct + lr and the
// eight columns 32 kg + (e & 4 ? 16 : 0) + 4 lg + (e & 3), e = 0..7, as 16 contiguous bytes, lane after
// lane.  Six fragments cover the lower triangle: (ct, kg) = (0,0) (1,0) (2,0) (2,1) (3,0) (3,1).  T is the
// A operand of U = T Z; P is the B operand P^T of O^T += U^T P^T.  Then four gate vectors of C floats.
constexpr int NFRAG = 6;
constexpr int kFragBytes = 64 * 16;
constexpr int kBlkT = 0, kBlkP = NFRAG * kFragBytes, kBlkVec = 2 * NFRAG * kFragBytes;
enum { PV_EG, PV_BETA, PV_EGC_G, PV_EGC, PV_N };
constexpr int kBlockBytes = kBlkVec + PV_N * C * 4;  // 13,312
static_assert(kBlockBytes == kTwoPassBlockBytes, "block size the host sizes the workspace with");
__host__ __device__ constexpr int frag_index(int ct, int kg) { return ct < 2 ? ct : 2 * ct - 2 + kg; }

// Chunk slot of (sequence n, chunk c): batch rows n * ceil(T / C) + c; packed sequences chunk_base[n] + c.
__device__ __forceinline__ int chunk_slot(const int32_t* chunk_base, int n, int c, int nch_row) {
  return (chunk_base ? chunk_base[n] : n * nch_row) + c;
}

// Exclusive prefix sum of the packed sequences' chunk counts: out[n] is sequence n's first chunk slot,
// out[N] the number of slots.  One workgroup; each thread sums a run of sequences.
__global__ __launch_bounds__(1024) void chunk_base_kernel(const int32_t* cu, int N, int32_t* out) {
  __shared__ int part[1024];
  const int per = (N + 1023) / 1024;
  const int lo = min(N, static_cast<int>(threadIdx.x) * per), hi = min(N, lo + per);
  int sum = 0;
  for (int n = lo; n < hi; ++n) sum += (cu[n + 1] - cu[n] + C - 1) / C;
  part[threadIdx.x] = sum;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int v = threadIdx.x >= static_cast<unsigned>(off) ? part[threadIdx.x - off] : 0;
    __syncthreads();
    part[threadIdx.x] += v;
    __syncthreads();
  }
  int base = threadIdx.x ? part[threadIdx.x - 1] : 0;
  if (threadIdx.x == 0) out[0] = 0;
  for (int n = lo; n < hi; ++n) {
    base += (cu[n + 1] - cu[n] + C - 1) / C;
    out[n + 1] = base;
  }
}

// ---------------------------------------------------------------- pass 1: chunk-local operands
struct PrepParams {
  const bf16 *q, *k;
  const float *g, *beta;
  const int32_t* cu;          // null: batch rows
  const int32_t* chunk_base;  // packed sequences: [N + 1] slots (chunk_base_kernel)
  unsigned char* blocks;      // [slot][Hv] workspace blocks
  int T, N, Hqk, Hv, nch_row, slots;
};

// Gram tiles (ti >= tj) of prep wave W: every wave forms both K K^T and Q K^T of its tiles.
template <int W> struct PrepTiles;
template <> struct PrepTiles<0> { static constexpr int n = 3, ti[3] = {3, 3, 3}, tj[3] = {0, 1, 2}; };
template <> struct PrepTiles<1> { static constexpr int n = 2, ti[3] = {2, 2, 0}, tj[3] = {0, 1, 0}; };
template <> struct PrepTiles<2> { static constexpr int n = 3, ti[3] = {1, 1, 2}, tj[3] = {0, 1, 2}; };
template <> struct PrepTiles<3> { static constexpr int n = 2, ti[3] = {0, 3, 0}, tj[3] = {0, 3, 0}; };

__global__ __launch_bounds__(256) void prep_kernel(PrepParams p) {
  __shared__ __attribute__((aligned(16))) float sA[C * LDF];  // A (strictly lower), fp32
  __shared__ __attribute__((aligned(16))) float sT[C * LDF];  // T = (I + A)^-1 (zero above the diagonal blocks)
  __shared__ __attribute__((aligned(16))) float sAd[4 * 16 * LDA];  // diagonal blocks of A, transposed
  __shared__ __attribute__((aligned(16))) float sVec[VEC_N * C];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lg = lane >> 4, lr = lane & 15;
  const int hq = blockIdx.x % p.Hqk;
  const int slot = blockIdx.x / p.Hqk;
  // slot -> (sequence n, chunk c)
  int n, c;
  if (p.cu) {
    if (slot >= p.chunk_base[p.N]) return;
    int lo = 0, hi = p.N - 1;  // the last n with chunk_base[n] <= slot (empty sequences share their base)
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (p.chunk_base[mid] <= slot) lo = mid; else hi = mid - 1;
    }
    n = lo;
    c = slot - p.chunk_base[n];
  } else {
    n = slot / p.nch_row;
    c = slot % p.nch_row;
    if (n >= p.N) return;
  }
  const int bos = p.cu ? p.cu[n] : n * p.T;
  const int eos = p.cu ? p.cu[n + 1] : bos + p.T;
  const int cs = bos + c * C, Lc = min(C, eos - cs);
  const int rep = p.Hv / p.Hqk;

  // blocks above the diagonal blocks of T stay zero
  for (int i = tid; i < C * C / 4; i += 256) {
    const int r = i / (C / 4), c4 = 4 * (i % (C / 4));
    if (c4 >= 16 * (r / 16 + 1)) *reinterpret_cast<floatx4*>(sT + r * LDF + c4) = zero4();
  }

  // Gram tiles from K and Q rows read straight from memory (rows past the end of the sequence read its
  // last token: finite, and their gates are masked to g = 0, beta = 0 below).
  const size_t qk_tok = static_cast<size_t>(p.Hqk) * D;
  auto row_frag = [&](const bf16* base, int t, int kgi) __attribute__((always_inline)) {
    const int r = min(16 * t + lr, Lc - 1);
    return *reinterpret_cast<const bf16x8*>(base + static_cast<size_t>(cs + r) * qk_tok + hq * D + 32 * kgi + 8 * lg);
  };
  floatx4 kk[3], qk[3];
  auto gram = [&](auto wtag) __attribute__((always_inline)) {
    using GT = PrepTiles<decltype(wtag)::value>;
    bf16x8 rk[KGK][4], rq[KGK][4];
#pragma unroll
    for (int kgi = 0; kgi < KGK; ++kgi)
#pragma unroll
      for (int t = 0; t < GT::n; ++t) {
        rk[kgi][GT::ti[t]] = row_frag(p.k, GT::ti[t], kgi);
        rk[kgi][GT::tj[t]] = row_frag(p.k, GT::tj[t], kgi);
        rq[kgi][GT::ti[t]] = row_frag(p.q, GT::ti[t], kgi);
      }
#pragma unroll
    for (int t = 0; t < 3; ++t) kk[t] = qk[t] = zero4();
#pragma unroll
    for (int kgi = 0; kgi < KGK; ++kgi)
#pragma unroll
      for (int t = 0; t < GT::n; ++t) {  // lane holds X[16 ti + lr][16 tj + 4 lg + s]
        Mma<bf16>::mma(kk[t], rk[kgi][GT::tj[t]], rk[kgi][GT::ti[t]]);
        Mma<bf16>::mma(qk[t], rk[kgi][GT::tj[t]], rq[kgi][GT::ti[t]]);
      }
  };
  switch (wave) {
    case 0: gram(std::integral_constant<int, 0>()); break;
    case 1: gram(std::integral_constant<int, 1>()); break;
    case 2: gram(std::integral_constant<int, 2>()); break;
    default: gram(std::integral_constant<int, 3>()); break;
  }

  // A and P of this wave's tiles for value head h: P to the workspace, A to LDS.
  auto tiles_out = [&](auto wtag, unsigned char* blk) __attribute__((always_inline)) {
    using GT = PrepTiles<decltype(wtag)::value>;
    const float* beta = sVec + VEC_BETA * C;
#pragma unroll
    for (int t = 0; t < GT::n; ++t) {
      const int ti = GT::ti[t], tj = GT::tj[t], i = 16 * ti + lr;
      const floatx4 dd = decay_tile(sVec, ti, tj, lg, lr);
      const float bi = beta[i];
      floatx4 a, pv;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int j = 16 * tj + 4 * lg + s;
        a[s] = j < i ? bi * dd[s] * kk[t][s] : 0.f;
        pv[s] = dd[s] * qk[t][s];
      }
      bf16x4* pf = reinterpret_cast<bf16x4*>(blk + kBlkP + frag_index(ti, tj >> 1) * kFragBytes + lane * 16) + (tj & 1);
      *pf = pack4<bf16>(pv[0], pv[1], pv[2], pv[3]);
      if (ti == 0 && tj == 0) *(pf + 1) = pack4<bf16>(0.f, 0.f, 0.f, 0.f);  // tile (0, 1): above the diagonal
      if (ti == 2 && tj == 2) *(pf + 1) = pack4<bf16>(0.f, 0.f, 0.f, 0.f);  // tile (2, 3)
      *reinterpret_cast<floatx4*>(sA + i * LDF + 16 * tj + 4 * lg) = a;
      if (ti == tj) {
#pragma unroll
        for (int s = 0; s < 4; ++s) sAd[(ti * 16 + 4 * lg + s) * LDA + lr] = a[s];
      }
    }
  };

  for (int hh = 0; hh < rep; ++hh) {
    const int h = hq * rep + hh;
    unsigned char* blk = p.blocks + (static_cast<size_t>(slot) * p.Hv + h) * kBlockBytes;
    if (wave == 3) {  // gates: inclusive prefix sum of g over the chunk, decay factors
      const bool live = lane < Lc;  // tokens past the end act as g = 0, beta = 0 (exact no-ops)
      const size_t gi = static_cast<size_t>(cs + min(lane, Lc - 1)) * p.Hv + h;
      const float gv = live ? p.g[gi] : 0.f;
      const float bt = live ? p.beta[gi] : 0.f;
      const float Gl = wave_inclusive_sum(gv) * kLog2e;
      const float GlC = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, Gl), 63));
      const float eg = __builtin_amdgcn_exp2f(Gl), egcg = __builtin_amdgcn_exp2f(GlC - Gl);
      const float egc = __builtin_amdgcn_exp2f(GlC);
      sVec[VEC_EG * C + lane] = eg;
      sVec[VEC_BETA * C + lane] = bt;
      sVec[VEC_GL * C + lane] = Gl;
#pragma unroll
      for (int b = 0; b < 3; ++b) {  // exp(-|G - G_r|), r = 16b + 15
        const float Gr = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, Gl), 16 * b + 15));
        sVec[(VEC_E0 + b) * C + lane] = __builtin_amdgcn_exp2f(lane <= 16 * b + 15 ? Gr - Gl : Gl - Gr);
      }
      float* pv = reinterpret_cast<float*>(blk + kBlkVec);
      pv[PV_EG * C + lane] = eg;
      pv[PV_BETA * C + lane] = bt;
      pv[PV_EGC_G * C + lane] = egcg;
      pv[PV_EGC * C + lane] = egc;
    }
    __syncthreads();
    switch (wave) {
      case 0: tiles_out(std::integral_constant<int, 0>(), blk); break;
      case 1: tiles_out(std::integral_constant<int, 1>(), blk); break;
      case 2: tiles_out(std::integral_constant<int, 2>(), blk); break;
      default: tiles_out(std::integral_constant<int, 3>(), blk); break;
    }
    __syncthreads();
    {  // wave w inverts diagonal block w of I + A (four lanes per column)
      const int cc = lane >> 2, q = lane & 3;
      floatx4 x;
#pragma unroll
      for (int t = 0; t < 4; ++t) x[t] = (4 * q + t == cc) ? 1.f : 0.f;
      unit_lower_inverse_column(x, sAd + wave * 16 * LDA, LDA, q, std::make_integer_sequence<int, 15>());
#pragma unroll
      for (int t = 0; t < 4; ++t) sT[(16 * wave + 4 * q + t) * LDF + 16 * wave + cc] = x[t];
    }
    __syncthreads();
    {  // wave w: the blocks of column block w below the diagonal,
       //   T_iw = -T_ii (A_iw T_ww + sum_{w<k<i} A_ik T_kw),
       // in fp32 on the matrix cores; each new block stays in registers as the B operand of the next.
      const int w = wave;
      floatx4 tw[4];  // T_kw in the accumulator layout (lane holds T_kw[4 lg + s][lr]), k > w
      floatx4 tww;    // T_ww as a B operand: T_ww[4 lg + s][lr]
#pragma unroll
      for (int s = 0; s < 4; ++s) tww[s] = sT[(16 * w + 4 * lg + s) * LDF + 16 * w + lr];
#pragma unroll
      for (int i = 1; i < 4; ++i) {
        if (i <= w) continue;
        floatx4 x = zero4();
        Mma<float>::mma(x, *reinterpret_cast<const floatx4*>(sA + (16 * i + lr) * LDF + 16 * w + 4 * lg), tww);
#pragma unroll
        for (int k = 1; k < 3; ++k)
          if (k > w && k < i)
            Mma<float>::mma(x, *reinterpret_cast<const floatx4*>(sA + (16 * i + lr) * LDF + 16 * k + 4 * lg), tw[k]);
        floatx4 t = zero4();
        Mma<float>::mma(t, *reinterpret_cast<const floatx4*>(sT + (16 * i + lr) * LDF + 16 * i + 4 * lg), x);
        tw[i] = -t;
#pragma unroll
        for (int s = 0; s < 4; ++s) sT[(16 * i + 4 * lg + s) * LDF + 16 * w + lr] = tw[i][s];
      }
    }
    __syncthreads();
    // T fragments to the workspace (bf16): 6 x 64 lanes of 16 bytes
    for (int it = tid; it < NFRAG * 64; it += 256) {
      const int f = it >> 6, l = it & 63;
      const int ct = f < 2 ? f : (f + 2) >> 1, kg = f < 2 ? 0 : (f & 1);
      const float* row = sT + (16 * ct + (l & 15)) * LDF + 32 * kg + 4 * (l >> 4);
      const floatx4 a = *reinterpret_cast<const floatx4*>(row), b = *reinterpret_cast<const floatx4*>(row + 16);
      bf16x8 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[e] = static_cast<bf16>(a[e]);
        v[4 + e] = static_cast<bf16>(b[e]);
      }
      *reinterpret_cast<bf16x8*>(blk + kBlkT + it * 16) = v;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- pass 2: the sequential scan
constexpr int BV = 32;      // state columns per workgroup
constexpr int NCW = 2;      // recurrence wavefronts (one 16-column tile each), as many output wavefronts
constexpr int NWAVES = NP + 2 * NCW;

struct ScanLayout {
  static constexpr size_t sK = 0;
  static constexpr size_t sQ = sK + 2 * C * LDK;
  static constexpr size_t sV = sQ + 2 * C * LDK;     // [C][BV] swizzled (swz_off<BV>)
  static constexpr size_t sKn = sV + 2 * C * BV;     // column-read copy of K (kn_piece)
  static constexpr size_t sBlk = sKn + 2 * C * D;    // the workspace block: T, P fragments, gate vectors
  static constexpr size_t stage_bytes = sBlk + kBlockBytes;
  static constexpr size_t oMx = 2 * stage_bytes;     // per recurrence wave: the state as bf16 operands
  static constexpr size_t oUx = oMx + NCW * KGK * 64 * 16;  // per recurrence wave: U as bf16 operands
  static constexpr size_t bytes = oUx + NCW * 2 * 64 * 16;
  static_assert(stage_bytes % 16 == 0 && sBlk % 16 == 0, "16-byte aligned LDS regions");
};
static_assert(ScanLayout::bytes <= 160 * 1024, "LDS budget of one gfx950 compute unit");

struct ScanParams {
  const bf16 *q, *k, *v;
  const float* h0;
  const int32_t* cu;
  const int32_t* chunk_base;
  const int32_t* order;
  const unsigned char* blocks;
  bf16* o;
  float* hT;
  int T, Hqk, Hv, nslices, grp, ngroups, nch_row;
  float scale;
};

__global__ __launch_bounds__(64 * NWAVES) void scan_kernel(ScanParams p) {
  using L = ScanLayout;
  using MM = Mma<bf16>;
  using frag = bf16x8;
  constexpr int KT = D / 16;  // key tiles of the state
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool stager = wave < NP;
  const bool chain = !stager && wave < NP + NCW;  // else an output wave
  const int lg = lane >> 4, lr = lane & 15;

  // Workgroup -> (unit, slice): the slices of a unit, and the value heads of one q/k head, get ids 8
  // apart, so they run on one XCD and share its L2 (they read the same K and Q).
  const int xcd = blockIdx.x & 7;
  const int rest = blockIdx.x >> 3;
  const int slice = rest % p.nslices;
  const int member = (rest / p.nslices) % p.grp;
  const int grp = (rest / p.nslices / p.grp) * 8 + xcd;
  if (grp >= p.ngroups) return;
  const int unit = grp * p.grp + member;  // = sequence * Hv + h
  const int h = unit % p.Hv;
  const int n = p.order ? p.order[unit / p.Hv] : unit / p.Hv;
  const int hq = h / (p.Hv / p.Hqk);
  const int bos = p.cu ? p.cu[n] : n * p.T;
  const int eos = p.cu ? p.cu[n + 1] : bos + p.T;
  const int nch = (eos - bos + C - 1) / C;
  const int col0 = slice * BV;
  const int cw = stager ? 0 : (wave - NP) % NCW;  // recurrence wave index (an output wave: its partner's)
  const int wcol = col0 + 16 * cw;
  const size_t qk_tok = static_cast<size_t>(p.Hqk) * D, v_tok = static_cast<size_t>(p.Hv) * D;
  auto stage = [&](int s) __attribute__((always_inline)) { return smem + s * L::stage_bytes; };
  frag* sMx = reinterpret_cast<frag*>(smem + L::oMx) + cw * KGK * 64;
  frag* sUx = reinterpret_cast<frag*>(smem + L::oUx) + cw * 2 * 64;

  if (stager) {
    // ---------------------------------------------------------- stagers: chunk c + 1 into LDS, c + 2 loaded
    ChunkRegs<bf16, D, BV> pre;
    constexpr int BIT = (kBlockBytes / 16 + PTHREADS - 1) / PTHREADS;  // workspace pieces per thread
    frag blk[BIT];
    auto load = [&](int c) __attribute__((always_inline)) {
      const int cs = bos + c * C;
      const size_t tq = static_cast<size_t>(cs) * qk_tok + static_cast<size_t>(hq) * D;
      const size_t tv = static_cast<size_t>(cs) * v_tok + static_cast<size_t>(h) * D + col0;
      pre.load_kqv(p.k + tq, p.q + tq, p.v + tv, static_cast<uint32_t>(qk_tok * 2), static_cast<uint32_t>(v_tok * 2),
                   min(C, eos - cs), tid);
      const frag* b = reinterpret_cast<const frag*>(
          p.blocks + (static_cast<size_t>(chunk_slot(p.chunk_base, n, c, p.nch_row)) * p.Hv + h) * kBlockBytes);
#pragma unroll
      for (int i = 0; i < BIT; ++i) blk[i] = b[min(tid + i * PTHREADS, kBlockBytes / 16 - 1)];
    };
    auto store = [&](int s) __attribute__((always_inline)) {
      unsigned char* S = stage(s);
      pre.store(reinterpret_cast<bf16*>(S + L::sK), reinterpret_cast<bf16*>(S + L::sQ),
                reinterpret_cast<bf16*>(S + L::sV), reinterpret_cast<bf16*>(S + L::sKn), LDK, BV, tid);
      frag* d = reinterpret_cast<frag*>(S + L::sBlk);
#pragma unroll
      for (int i = 0; i < BIT; ++i)
        if (tid + i * PTHREADS < kBlockBytes / 16) d[tid + i * PTHREADS] = blk[i];
    };
    __builtin_amdgcn_s_setprio(1);
    if (nch > 0) {
      load(0);
      store(0);
      if (nch > 1) load(1);
    }
    lds_barrier();
    for (int c = 0; c < nch; ++c) {
      if (c + 1 < nch) {
        store((c + 1) & 1);
        if (c + 2 < nch) load(c + 2);
      }
      lds_barrier();
      lds_barrier();
    }
    return;
  }

  // ------------------------------------------------------------ recurrence and output wavefronts
  // Ms[a] holds M[state_row(a, lg, s)][wcol + lr], s = 0..3 (recurrence waves only).
  floatx4 Ms[KT];
  frag mfr[KGK];  // the state as matrix-core operands (bf16), per chunk
  const size_t sbase = (static_cast<size_t>(n) * p.Hv + h) * D * D;
  const int slane = MM::state_row(0, lg, 0) * D + wcol + lr;
  auto state_operands = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int kgi = 0; kgi < KGK; ++kgi) {
      mfr[kgi] = MM::chain(Ms[2 * kgi], Ms[2 * kgi + 1]);
      sMx[kgi * 64 + lane] = mfr[kgi];
    }
  };
  if (chain) {
    const float* h0 = p.h0 + sbase;
#pragma unroll
    for (int a = 0; a < KT; ++a)
#pragma unroll
      for (int s = 0; s < 4; ++s) Ms[a][s] = p.h0 ? h0[slane + MM::state_row(a, 0, s) * D] : 0.f;
    __builtin_amdgcn_s_setprio(2);
    state_operands();
    lds_barrier();
    for (int c = 0; c < nch; ++c) {
      const unsigned char* S = stage(c & 1);
      const bf16* sK = reinterpret_cast<const bf16*>(S + L::sK);
      const bf16* sV = reinterpret_cast<const bf16*>(S + L::sV);
      const float* vec = reinterpret_cast<const float*>(S + L::sBlk + kBlkVec);
      const frag* sT = reinterpret_cast<const frag*>(S + L::sBlk + kBlkT);
      // Z = diag(beta) (V - diag(exp G) K M)
      floatx4 Z[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) Z[r] = zero4();
#pragma unroll
      for (int kgi = 0; kgi < KGK; ++kgi)
#pragma unroll
        for (int r = 0; r < 4; ++r) MM::mma(Z[r], lds_frag(sK + (16 * r + lr) * LDK, kgi, lane), mfr[kgi]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bf16x4 v4 = swz_col4<BV>(sV, 16 * r, 16 * cw, lane);
        const floatx4 eg = *reinterpret_cast<const floatx4*>(vec + PV_EG * C + 16 * r + 4 * lg);
        const floatx4 bt = *reinterpret_cast<const floatx4*>(vec + PV_BETA * C + 16 * r + 4 * lg);
#pragma unroll
        for (int s = 0; s < 4; ++s) Z[r][s] = bt[s] * (static_cast<float>(v4[s]) - eg[s] * Z[r][s]);
      }
      // U = T Z; U goes to the output wave as operands
      const frag zf0 = MM::chain(Z[0], Z[1]), zf1 = MM::chain(Z[2], Z[3]);
      floatx4 U[4];
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        U[ct] = zero4();
        MM::mma(U[ct], sT[frag_index(ct, 0) * 64 + lane], zf0);
        if (ct >= 2) MM::mma(U[ct], sT[frag_index(ct, 1) * 64 + lane], zf1);
      }
      sUx[lane] = MM::chain(U[0], U[1]);
      sUx[64 + lane] = MM::chain(U[2], U[3]);
      lds_barrier();
      // M <- exp(G_C) M + K^T diag(exp(G_C - G)) U
      int olane;
      asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(olane));
      const KnCols<D> kcols(reinterpret_cast<const bf16*>(S + L::sKn), olane);
      const float eGC = vec[PV_EGC * C];
#pragma unroll
      for (int r = 0; r < 4; ++r) U[r] *= *reinterpret_cast<const floatx4*>(vec + PV_EGC_G * C + 16 * r + 4 * lg);
#pragma unroll
      for (int a = 0; a < KT; ++a) Ms[a] *= eGC;
#pragma unroll
      for (int kgi = 0; kgi < 2; ++kgi) {
        const frag bu = MM::chain(U[2 * kgi], U[2 * kgi + 1]);
#pragma unroll
        for (int a = 0; a < KT; ++a) {
          const bf16* pa = kcols.tile(a) + 32 * kgi * D;
          const frag af = __builtin_shufflevector(tr_read(pa), tr_read(pa + 16 * D), 0, 1, 2, 3, 4, 5, 6, 7);
          MM::mma(Ms[a], af, bu);
        }
      }
      state_operands();
      lds_barrier();
    }
    if (p.hT) {
      float* hT = p.hT + sbase;
#pragma unroll
      for (int a = 0; a < KT; ++a)
#pragma unroll
        for (int s = 0; s < 4; ++s) hT[slane + MM::state_row(a, 0, s) * D] = Ms[a][s];
    }
    return;
  }

  // output waves: O^T = scale (diag-scaled (Q M)^T + U^T P^T), lane holds O[16 ct + lr][wcol + 4 lg + s]
  lds_barrier();
  for (int c = 0; c < nch; ++c) {
    const unsigned char* S = stage(c & 1);
    const bf16* sQ = reinterpret_cast<const bf16*>(S + L::sQ);
    const float* vec = reinterpret_cast<const float*>(S + L::sBlk + kBlkVec);
    const frag* sP = reinterpret_cast<const frag*>(S + L::sBlk + kBlkP);
#pragma unroll
    for (int kgi = 0; kgi < KGK; ++kgi) mfr[kgi] = sMx[kgi * 64 + lane];
    floatx4 Ot[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      Ot[ct] = zero4();
#pragma unroll
      for (int kgi = 0; kgi < KGK; ++kgi) MM::mma(Ot[ct], mfr[kgi], lds_frag(sQ + (16 * ct + lr) * LDK, kgi, lane));
      Ot[ct] *= vec[PV_EG * C + 16 * ct + lr];
    }
    lds_barrier();
    const frag u0 = sUx[lane], u1 = sUx[64 + lane];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      MM::mma(Ot[ct], u0, sP[frag_index(ct, 0) * 64 + lane]);
      if (ct >= 2) MM::mma(Ot[ct], u1, sP[frag_index(ct, 1) * 64 + lane]);
    }
    const int cs = bos + c * C, Lc = min(C, eos - cs);
    bf16* orow = p.o + static_cast<size_t>(cs + lr) * v_tok + static_cast<size_t>(h) * D + wcol + 4 * lg;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      if (16 * ct + lr < Lc) {
        const floatx4 ov = Ot[ct] * p.scale;
        *reinterpret_cast<bf16x4*>(orow + static_cast<size_t>(16 * ct) * v_tok) = pack4<bf16>(ov[0], ov[1], ov[2], ov[3]);
      }
    }
    lds_barrier();
  }
}

}  // namespace

hipError_t launch_chunk_base(const int32_t* cu, int num_seqs, int32_t* chunk_base, hipStream_t stream) {
  chunk_base_kernel<<<dim3(1), dim3(1024), 0, stream>>>(cu, num_seqs, chunk_base);
  return hipGetLastError();
}

hipError_t launch_two_pass(const PrefillArgs& a, hipStream_t stream) {
  const bool packed = a.cu_seqlens != nullptr;
  const TwoPassParts w = two_pass_parts(a.batch, a.seqlen, a.num_seqs, packed, a.Hv);
  unsigned char* ws = static_cast<unsigned char*>(a.workspace);
  const int32_t* chunk_base = nullptr;
  const int32_t* order = nullptr;
  if (packed) {
    int32_t* cb = reinterpret_cast<int32_t*>(ws + w.chunk_base);
    hipError_t e = launch_chunk_base(a.cu_seqlens, a.num_seqs, cb, stream);
    if (e != hipSuccess) return e;
    chunk_base = cb;
    if (order_workspace_bytes(a.num_seqs)) {
      int32_t* ord = reinterpret_cast<int32_t*>(ws + w.order);
      hipError_t e = launch_order(a.cu_seqlens, a.num_seqs, ord, stream);
      if (e != hipSuccess) return e;
      order = ord;
    }
  }
  const int nch_row = (a.seqlen + C - 1) / C;
  PrepParams pp;
  pp.q = static_cast<const bf16*>(a.q);
  pp.k = static_cast<const bf16*>(a.k);
  pp.g = a.g;
  pp.beta = a.beta;
  pp.cu = a.cu_seqlens;
  pp.chunk_base = chunk_base;
  pp.blocks = ws + w.blocks;
  pp.T = a.seqlen;
  pp.N = a.num_seqs;
  pp.Hqk = a.Hqk;
  pp.Hv = a.Hv;
  pp.nch_row = nch_row;
  pp.slots = static_cast<int>(w.slots);
  if (w.slots > 0) prep_kernel<<<dim3(static_cast<unsigned>(w.slots * a.Hqk)), dim3(256), 0, stream>>>(pp);

  ScanParams sp;
  sp.q = pp.q;
  sp.k = pp.k;
  sp.v = static_cast<const bf16*>(a.v);
  sp.h0 = a.initial_state;
  sp.cu = a.cu_seqlens;
  sp.chunk_base = chunk_base;
  sp.order = order;
  sp.blocks = ws + w.blocks;
  sp.o = static_cast<bf16*>(a.o);
  sp.hT = a.final_state;
  sp.T = a.seqlen;
  sp.Hqk = a.Hqk;
  sp.Hv = a.Hv;
  sp.nslices = D / BV;
  sp.grp = a.Hv / a.Hqk;
  sp.ngroups = a.num_seqs * a.Hqk;
  sp.nch_row = nch_row;
  sp.scale = a.scale;
  if (sp.ngroups == 0) return hipGetLastError();
  const int groups_pad = (sp.ngroups + 7) / 8 * 8;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&scan_kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(ScanLayout::bytes));
  if (e != hipSuccess) return e;
  scan_kernel<<<dim3(groups_pad * sp.grp * sp.nslices), dim3(64 * NWAVES), ScanLayout::bytes, stream>>>(sp);
  return hipGetLastError();
}

}  // namespace gdn

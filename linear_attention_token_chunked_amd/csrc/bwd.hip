// Backward pass of the gated delta rule, chunked, gfx950: the gradients of a
// prefill with respect to q, k, v, g, beta and the initial state.
//
// Training cost is one of the axes the report on "On the Design of
// Qwen3.8-Next Architecture" weighs every change on (paper page, Abstract); the
// recurrence is the one of cue 14 of the podcast transcript on it.  Per chunk of
// C = 64 tokens starting from state M (dk x dv, the stored layout), with G the
// in-chunk inclusive cumsum of g, gam = exp(G), kf = exp(G_C - G), s = scale:
//   P = lower_incl(s exp(G_i - G_j) Q K^T),  A = strict_lower(beta_i exp(G_i - G_j) K K^T),
//   Z = diag(beta) (V - diag(gam) K M),  U = (I + A)^-1 Z,
//   O = s diag(gam) Q M + P U,  M' = gam_C M + K^T diag(kf) U.
// Differentiating that chunk form with dO and dM' (the gradient of the state
// after the chunk) given:
//   dU = P^T dO + diag(kf) K dM',   dZ = (I + A)^-T dU,
//   dM = gam_C dM' + s Q^T diag(gam) dO - K^T diag(beta gam) dZ,
//   dV = diag(beta) dZ,  dP = lower_incl(dO U^T),  dA = strict_lower(-dZ U^T),
//   dq = s diag(gam) dO M^T + (dP * s exp(G_i - G_j)) K,
//   dk = -diag(beta gam) dZ M^T + diag(kf) U dM'^T + (dP * sG)^T Q + (D + D^T) K,
//        D = dA * beta_i exp(G_i - G_j),
//   dbeta_i = dZ_i . (V_i - gam_i (K M)_i) + sum_j dA_ij exp(G_i - G_j) (K K^T)_ij,
// and dG from every place G enters (gam, kf, gam_C and the two decay masks),
// summed into dg by a reverse cumsum inside the chunk.  Three kernels:
//   1. the forward prefill in its saving variant keeps each chunk's starting
//      state and U (in the input's element type: the operands the products use);
//   2. dstate_kernel walks each (sequence, value head, 32-column slice of dv)
//      backwards over its chunks, holding dM in registers: it keeps dM' and dZ
//      per chunk and leaves dM of the first chunk as the initial state's gradient;
//   3. dlocal_kernel forms every per-token gradient of one chunk, all chunks in
//      parallel, one workgroup per query/key head walking the value heads that
//      share it (their dq and dk summed in registers).
// Every sum is taken in a fixed order and every output element is written once
// (no atomics), so a call's gradients do not depend on scheduling: the same
// inputs give bitwise the same gradients.
// Products run on the matrix cores over 16-wide k-steps with operands in LDS
// (bf16 inputs: bf16 operands, fp32 accumulation; fp32 inputs: fp32 throughout).
// Workgroup barriers order LDS only (lds_barrier): the stores to the workspace
// and the outputs, which no thread of the same kernel reads, stay in flight
// across them.
#include "device_common.hpp"
#include "launch.hpp"

namespace gdn {
namespace {

constexpr int C = 64;  // chunk length

// ------------------------------------------------------------------ helpers
// Lane (g, lr) gets X[lr][4g + e], e = 0..3: a row-major tile read along its rows.
template <class T>
__device__ __forceinline__ typename Vec4<T>::type row4(const T* X, int ld, int lane) {
  return *reinterpret_cast<const typename Vec4<T>::type*>(X + (lane & 15) * ld + 4 * (lane >> 4));
}

// acc (16x16 accumulator tile) += sum_{k < K} opA(m, k) opB(n, k), K a multiple
// of 16, where opA(m, k) = TA ? A[k][m] : A[m][k] and likewise for B (row
// strides lda, ldb; A and B point at element (0, 0) of the operands).
template <class T, bool TA, bool TB, int K>
__device__ __forceinline__ void tile_mm(floatx4& acc, const T* A, int lda, const T* B, int ldb, int lane) {
#pragma unroll
  for (int k0 = 0; k0 < K; k0 += 16) {
    const auto fa = TA ? lds_col4<T>(A + k0 * lda, lda, 0, 0, lane) : row4<T>(A + k0, lda, lane);
    const auto fb = TB ? lds_col4<T>(B + k0 * ldb, ldb, 0, 0, lane) : row4<T>(B + k0, ldb, lane);
    Mma16<T>::mma(acc, fa, fb);
  }
}

// The same product when both operands are read along their rows (no
// transposes): whole k-groups of the wide matrix-core instruction
// (bf16: 16x16x32, 16-byte row reads), K a multiple of Mma<T>::KG.
template <class T, int K>
__device__ __forceinline__ void tile_mm_nn(floatx4& acc, const T* A, int lda, const T* B, int ldb, int lane) {
  static_assert(K % Mma<T>::KG == 0, "whole k-groups");
  const T* ar = A + (lane & 15) * lda;
  const T* br = B + (lane & 15) * ldb;
#pragma unroll
  for (int kg = 0; kg < K / Mma<T>::KG; ++kg) Mma<T>::mma(acc, lds_frag<T>(ar, kg, lane), lds_frag<T>(br, kg, lane));
}

// A B operand read once and used for several output tiles: the k-groups of
// rows (lane & 15) of B (row reads), or the 16-wide k-steps of columns
// (lane & 15) of B (column reads).
template <class T, int K>
struct RowFrags {
  typename Mma<T>::frag f[K / Mma<T>::KG];
  __device__ __forceinline__ RowFrags(const T* B, int ldb, int lane) {
#pragma unroll
    for (int kg = 0; kg < K / Mma<T>::KG; ++kg) f[kg] = lds_frag<T>(B + (lane & 15) * ldb, kg, lane);
  }
};
template <class T, int K>
struct ColFrags {
  typename Vec4<T>::type f[K / 16];
  __device__ __forceinline__ ColFrags(const T* B, int ldb, int lane) {
#pragma unroll
    for (int k = 0; k < K / 16; ++k) f[k] = lds_col4<T>(B + 16 * k * ldb, ldb, 0, 0, lane);
  }
};
template <class T, int K>
__device__ __forceinline__ void tile_mm_nn(floatx4& acc, const T* A, int lda, const RowFrags<T, K>& b, int lane) {
  const T* ar = A + (lane & 15) * lda;
#pragma unroll
  for (int kg = 0; kg < K / Mma<T>::KG; ++kg) Mma<T>::mma(acc, lds_frag<T>(ar, kg, lane), b.f[kg]);
}
template <class T, bool TA, int K>
__device__ __forceinline__ void tile_mm(floatx4& acc, const T* A, int lda, const ColFrags<T, K>& b, int lane) {
#pragma unroll
  for (int k = 0; k < K / 16; ++k) {
    const auto fa = TA ? lds_col4<T>(A + 16 * k * lda, lda, 0, 0, lane) : row4<T>(A + 16 * k, lda, lane);
    Mma16<T>::mma(acc, fa, b.f[k]);
  }
}

// Sum over the 16 lanes of a row group, in every lane of it (DPP row rotations:
// no LDS round trips).
__device__ __forceinline__ float sum16(float x) {
#define GDN_ROR_ADD(n) \
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x120 + (n), 0xf, 0xf, false))
  GDN_ROR_ADD(8);
  GDN_ROR_ADD(4);
  GDN_ROR_ADD(2);
  GDN_ROR_ADD(1);
#undef GDN_ROR_ADD
  return x;
}
// Sum over the 8 lanes of a half row group, in every lane of it (quad permutations
// l ^ 1 and l ^ 2, then the half-row mirror, which pairs the two quads).
__device__ __forceinline__ float sum8(float x) {
#define GDN_DPP_ADD(ctrl) \
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), ctrl, 0xf, 0xf, false))
  GDN_DPP_ADD(0xb1);
  GDN_DPP_ADD(0x4e);
  GDN_DPP_ADD(0x141);
#undef GDN_DPP_ADD
  return x;
}
__device__ __forceinline__ floatx4 vec4_at(const float* v) { return *reinterpret_cast<const floatx4*>(v); }
__device__ __forceinline__ float rdlane(float x, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
}

// Rows of a row-major tile held in registers on their way to LDS, as raw
// 16-byte pieces of EP elements: R rows of W columns, NT threads (rows >= L
// read as zero).
template <class T, int W, int NT, int R = C>
struct RowsInFlight {
  static constexpr int EP = 16 / sizeof(T), PR = W / EP, N = R * PR, IT = (N + NT - 1) / NT;
  typedef T piece __attribute__((ext_vector_type(EP)));
  piece v[IT];
  // src is the same for every lane; the per-lane part is a 32-bit byte offset
  // (at most 64 rows of at most 1 MB)
  __device__ __forceinline__ void load(const T* src, size_t ss, int L, int tid) {
    const char* base = reinterpret_cast<const char*>(src);
    const unsigned stride = static_cast<unsigned>(ss * sizeof(T));
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int i = tid + it * NT, t = i / PR, e = (i - t * PR) * EP;
      const unsigned off = static_cast<unsigned>(t) * stride + static_cast<unsigned>(e * sizeof(T));
      if (i < N && t < L) v[it] = *reinterpret_cast<const piece*>(base + off);
      else v[it] = piece{};
    }
  }
  __device__ __forceinline__ void store(T* dst, int ld, int tid) const {
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int i = tid + it * NT, t = i / PR, e = (i - t * PR) * EP;
      if (i < N) *reinterpret_cast<piece*>(dst + t * ld + e) = v[it];
    }
  }
};

// Per-chunk gate vectors, formed by one wavefront (lane = token): log2-scaled
// inclusive cumsum Gl, exp(G), exp(G_C - G), beta (tokens >= L act as g = 0,
// beta = 0), and exp(G_C) in vec[4C].
enum { V_GL, V_GAM, V_KF, V_BETA, V_N };
__device__ __forceinline__ void gate_vectors_from(float* vec, float gt, float bt, int lane) {
  const float Gl = wave_inclusive_sum(fmaxf(gt, kGateFloor)) * kLog2e;
  const float GlC = rdlane(Gl, 63);
  vec[V_GL * C + lane] = Gl;
  vec[V_GAM * C + lane] = __builtin_amdgcn_exp2f(Gl);
  vec[V_KF * C + lane] = __builtin_amdgcn_exp2f(GlC - Gl);
  vec[V_BETA * C + lane] = bt;
  if (lane == 0) vec[V_N * C] = __builtin_amdgcn_exp2f(GlC);
}
__device__ __forceinline__ void gate_vectors(float* vec, const float* g, const float* beta, size_t stride, int L,
                                             int lane) {
  const bool live = lane < L;
  gate_vectors_from(vec, live ? g[lane * stride] : 0.f, live ? beta[lane * stride] : 0.f, lane);
}

struct Seq {
  int bos, eos, cbase;  // token range and the global index of the first chunk
};
__device__ __forceinline__ Seq seq_of(const int32_t* cu, const int32_t* cpre, int T, int n) {
  if (cu) return Seq{cu[n], cu[n + 1], cpre[n]};
  return Seq{n * T, n * T + T, n * ((T + C - 1) / C)};
}

struct BwdParams {
  const void *q, *k, *v, *dout;
  const float *g, *beta, *dhT;
  const int32_t *cu, *cpre;
  const void *ck_state, *ck_u;  // chunk-start states, U (from the saving prefill), element type T
  void *dm, *dz;                // dM' per chunk, dZ per token (dstate_kernel), element type T
  float *dq, *dk, *dv, *dg, *dbeta, *dh0;
  int T, N, Hqk, Hv, chunk_bound;
  float scale;
};

// ------------------------------------------------------- state gradient scan
template <class T, int DK, int BV>
struct DsLayout {
  static constexpr int PAD = sizeof(T) == 2 ? 16 : 4;  // row padding: 32 bytes (bf16), 16 (fp32, to fit twice)
  static constexpr int LDK = DK + PAD, LDB = BV + PAD, LDC = C + (sizeof(T) == 2 ? 8 : PAD), LDD = 16 + PAD, LDF = BV + 4,
                       LDT = 20;
  // a chunk's inputs, double-buffered: K, Q, the dO slice, the gate vectors
  static constexpr int iK = 0;
  static constexpr int iQ = iK + C * LDK * sizeof(T);
  static constexpr int idO = iQ + C * LDK * sizeof(T);
  static constexpr int iVec = idO + C * LDB * sizeof(T);
  static constexpr int in_bytes = iVec + (V_N * C + 4) * 4;
  static constexpr int odOg = 2 * in_bytes;  // s gam dO
  static constexpr int odZ = odOg + C * LDB * sizeof(T);
  static constexpr int odZb = odZ + C * LDB * sizeof(T);  // -beta gam dZ
  static constexpr int odMn = odZb + C * LDB * sizeof(T);
  static constexpr int oP = odMn + DK * LDB * sizeof(T);
  static constexpr int oA = oP + C * LDC * sizeof(T);
  static constexpr int oTd = oA + C * LDC * sizeof(T);  // diagonal blocks of (I + A)^-1, row-major
  static constexpr int odU = oTd + 4 * 16 * LDD * sizeof(T);  // fp32
  static constexpr int oAt = odU + C * LDF * 4;               // fp32 diagonal blocks of A, transposed
  static constexpr int bytes = oAt + 4 * 16 * LDT * 4;
  static_assert(in_bytes % 16 == 0, "aligned buffers");
};

template <class T, int DK, int DV, int BV>
__global__ __launch_bounds__(512) void dstate_kernel(BwdParams p) {
  using L = DsLayout<T, DK, BV>;
  constexpr int LDK = L::LDK, LDB = L::LDB, LDC = L::LDC, LDD = L::LDD, LDF = L::LDF, LDT = L::LDT;
  constexpr int NW = 8, NT = 64 * NW;       // wavefronts, threads
  constexpr int NJ = BV / 16;               // column tiles of the slice (one solving wavefront each)
  constexpr int NST = 64 * (NW - NJ);       // threads that stage the next chunk meanwhile
  constexpr int NTL = (DK / 16) * NJ;       // dM tiles
  constexpr int NMT = (NTL + NW - 1) / NW;  // dM tiles per wavefront (some idle when NTL < NW)
  static_assert(NTL % NW == 0 || NTL < NW, "tiles split over the wavefronts");
  static_assert(4 * NJ <= NW, "one wavefront per dU tile");
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  T* sdOg = reinterpret_cast<T*>(smem + L::odOg);
  T* sdZ = reinterpret_cast<T*>(smem + L::odZ);
  T* sdZb = reinterpret_cast<T*>(smem + L::odZb);
  T* sdMn = reinterpret_cast<T*>(smem + L::odMn);
  T* sP = reinterpret_cast<T*>(smem + L::oP);
  T* sA = reinterpret_cast<T*>(smem + L::oA);
  T* sTd = reinterpret_cast<T*>(smem + L::oTd);
  float* sdU = reinterpret_cast<float*>(smem + L::odU);
  float* sAt = reinterpret_cast<float*>(smem + L::oAt);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lg = lane >> 4, lr = lane & 15;
  // workgroup -> (unit, slice); a unit's slices get ids 8 apart and so share one XCD's L2
  constexpr int NS = DV / BV;
  const int rest = blockIdx.x >> 3, slice = rest % NS;
  const int unit = (blockIdx.x & 7) + 8 * (rest / NS);
  if (unit >= p.N * p.Hv) return;
  const int col0 = slice * BV;
  const int n = unit / p.Hv, h = unit - n * p.Hv, hq = h / (p.Hv / p.Hqk);
  const Seq sq = seq_of(p.cu, p.cpre, p.T, n);
  const int nch = (sq.eos - sq.bos + C - 1) / C;
  const size_t sbase = static_cast<size_t>(unit) * DK * DV;
  const size_t qk_tok = static_cast<size_t>(p.Hqk) * DK, v_tok = static_cast<size_t>(p.Hv) * DV;

  // chunk c's inputs into buffer c & 1, by threads [t0, t0 + NTH) (gates: the first of their wavefronts)
  auto stage_in = [&](int c, int t0, auto nth) __attribute__((always_inline)) {
    constexpr int NTH = decltype(nth)::value;
    unsigned char* B = smem + (c & 1) * L::in_bytes;
    const int cs = sq.bos + c * C, Lc = min(C, sq.eos - cs), t = tid - t0;
    const size_t qo = static_cast<size_t>(cs) * qk_tok + static_cast<size_t>(hq) * DK;
    RowsInFlight<T, DK, NTH> rk, rq;
    RowsInFlight<T, BV, NTH> rdo;
    rk.load(static_cast<const T*>(p.k) + qo, qk_tok, Lc, t);
    rq.load(static_cast<const T*>(p.q) + qo, qk_tok, Lc, t);
    rdo.load(static_cast<const T*>(p.dout) + static_cast<size_t>(cs) * v_tok + static_cast<size_t>(h) * DV + col0, v_tok,
             Lc, t);
    if (t < 64) {
      const size_t gi = static_cast<size_t>(cs) * p.Hv + h;
      gate_vectors(reinterpret_cast<float*>(B + L::iVec), p.g + gi, p.beta + gi, p.Hv, Lc, lane);
    }
    rk.store(reinterpret_cast<T*>(B + L::iK), LDK, t);
    rq.store(reinterpret_cast<T*>(B + L::iQ), LDK, t);
    rdo.store(reinterpret_cast<T*>(B + L::idO), LDB, t);
  };
  // With bf16 inputs the staging wavefronts request a chunk's rows one iteration before they store
  // them (in the back-substitution phase, after storing the chunk requested the iteration before),
  // so the memory latency lands on no phase.  The fp32 instantiation has no registers to spare for
  // that and stages within the phase.
  constexpr bool AHEAD = sizeof(T) == 2;
  RowsInFlight<T, DK, NST> nk, nq;
  RowsInFlight<T, BV, NST> ndo;
  float ng = 0.f, nb = 0.f;
  auto stage_load = [&](int c) __attribute__((always_inline)) {
    const int cs = sq.bos + c * C, Lc = min(C, sq.eos - cs), t = tid - 64 * NJ;
    const size_t qo = static_cast<size_t>(cs) * qk_tok + static_cast<size_t>(hq) * DK;
    nk.load(static_cast<const T*>(p.k) + qo, qk_tok, Lc, t);
    nq.load(static_cast<const T*>(p.q) + qo, qk_tok, Lc, t);
    ndo.load(static_cast<const T*>(p.dout) + static_cast<size_t>(cs) * v_tok + static_cast<size_t>(h) * DV + col0, v_tok,
             Lc, t);
    if (t < 64) {
      const size_t gi = static_cast<size_t>(cs) * p.Hv + h;
      const bool live = lane < Lc;
      ng = live ? p.g[gi + lane * static_cast<size_t>(p.Hv)] : 0.f;
      nb = live ? p.beta[gi + lane * static_cast<size_t>(p.Hv)] : 0.f;
    }
  };
  auto stage_store = [&](int c) __attribute__((always_inline)) {
    unsigned char* B = smem + (c & 1) * L::in_bytes;
    const int t = tid - 64 * NJ;
    if (t < 64) gate_vectors_from(reinterpret_cast<float*>(B + L::iVec), ng, nb, lane);
    nk.store(reinterpret_cast<T*>(B + L::iK), LDK, t);
    nq.store(reinterpret_cast<T*>(B + L::iQ), LDK, t);
    ndo.store(reinterpret_cast<T*>(B + L::idO), LDB, t);
  };
  // dM' as matrix-core operands
  floatx4 dM[NMT];  // tile t = wave + NW i -> rows 16 (t / NJ), columns 16 (t % NJ)
  auto dm_to_lds = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NMT; ++i) {
      const int t = wave + NW * i, a = t / NJ, jc = t % NJ;
      if (t >= NTL) break;
#pragma unroll
      for (int r = 0; r < 4; ++r) sdMn[(16 * a + 4 * lg + r) * LDB + 16 * jc + lr] = from_float<T>(dM[i][r]);
    }
  };

#pragma unroll
  for (int i = 0; i < NMT; ++i) {
    const int t = wave + NW * i, a = t / NJ, jc = t % NJ;
    if (t >= NTL) break;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      dM[i][r] = p.dhT ? p.dhT[sbase + static_cast<size_t>(16 * a + 4 * lg + r) * DV + col0 + 16 * jc + lr] : 0.f;
  }
  if (nch > 0) stage_in(nch - 1, 0, std::integral_constant<int, NT>());
  if (AHEAD && nch > 1 && wave >= NJ) stage_load(nch - 2);
  dm_to_lds();
  lds_barrier();

  for (int c = nch - 1; c >= 0; --c) {
    const int cs = sq.bos + c * C, Lc = min(C, sq.eos - cs);
    const unsigned char* B = smem + (c & 1) * L::in_bytes;
    const T* sK = reinterpret_cast<const T*>(B + L::iK);
    const T* sQ = reinterpret_cast<const T*>(B + L::iQ);
    const T* sdO = reinterpret_cast<const T*>(B + L::idO);
    const float* vec = reinterpret_cast<const float*>(B + L::iVec);
    // -- dM' of this chunk to the workspace (from its operand copy, as whole 16-byte
    //    pieces); Gram tiles P and A (lower tiles), s gam dO
    {
      T* dmw = static_cast<T*>(p.dm) + (static_cast<size_t>(sq.cbase + c) * p.Hv + h) * DK * DV + col0;
      constexpr int EP = 16 / sizeof(T), PPR = BV / EP;  // elements per piece, pieces per row
      for (int i = tid; i < DK * PPR; i += NT) {
        const int r = i / PPR, e = (i - r * PPR) * EP;
        *reinterpret_cast<uint4*>(dmw + static_cast<size_t>(r) * DV + e) =
            *reinterpret_cast<const uint4*>(sdMn + r * LDB + e);
      }
    }
    {
      const float s = p.scale;
      for (int job = wave; job < 20; job += NW) {
        const int kind = job / 10, lt = job % 10;  // lower tile lt -> (ti, tj)
        const int ti = lt < 1 ? 0 : lt < 3 ? 1 : lt < 6 ? 2 : 3;
        const int tj = lt - ti * (ti + 1) / 2;
        floatx4 acc = zero4();
        tile_mm_nn<T, DK>(acc, (kind ? sK : sQ) + 16 * ti * LDK, LDK, sK + 16 * tj * LDK, LDK, lane);
        const int j = 16 * tj + lr, i0 = 16 * ti + 4 * lg;
        const floatx4 Gi = vec4_at(vec + V_GL * C + i0), bi = vec4_at(vec + V_BETA * C + i0);
        const float Gj = vec[V_GL * C + j];
        float val[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {  // branch-free: the masks are selects
          const int i = i0 + r;
          const float e = __builtin_amdgcn_exp2f(Gi[r] - Gj);
          val[r] = kind == 0 ? (j <= i ? s * e * acc[r] : 0.f) : (j < i ? bi[r] * e * acc[r] : 0.f);
        }
        T* dst = kind == 0 ? sP : sA;
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[(i0 + r) * LDC + j] = from_float<T>(val[r]);
        if (kind == 0 && ti != tj) {  // the tile above the diagonal is zero
#pragma unroll
          for (int r = 0; r < 4; ++r) sP[j * LDC + i0 + r] = from_float<T>(0.f);
        }
        if (kind == 1 && ti == tj)
          *reinterpret_cast<floatx4*>(sAt + (ti * 16 + lr) * LDT + 4 * lg) = floatx4{val[0], val[1], val[2], val[3]};
      }
      for (int i = tid; i < C * BV; i += NT) {
        const int t = i / BV, cc = i - t * BV;
        sdOg[t * LDB + cc] = from_float<T>(s * vec[V_GAM * C + t] * to_float(sdO[t * LDB + cc]));
      }
    }
    lds_barrier();
    // -- inverses of the diagonal blocks of I + A; dU = P^T dO + diag(kf) K dM'
    if (wave < 4) {
      const int cc = lane >> 2, q = lane & 3;
      floatx4 x;
#pragma unroll
      for (int t = 0; t < 4; ++t) x[t] = (4 * q + t == cc) ? 1.f : 0.f;
      unit_lower_inverse_column(x, sAt + wave * 16 * LDT, LDT, q, std::make_integer_sequence<int, 15>());
#pragma unroll
      for (int t = 0; t < 4; ++t) sTd[(wave * 16 + 4 * q + t) * LDD + cc] = from_float<T>(x[t]);
    }
    if (wave < 4 * NJ) {
      const int bt = wave / NJ, jc = wave % NJ;
      floatx4 acc = zero4(), acc2 = zero4();
      tile_mm<T, true, true, C>(acc, sP + 16 * bt, LDC, sdO + 16 * jc, LDB, lane);
      tile_mm<T, false, true, DK>(acc2, sK + 16 * bt * LDK, LDK, sdMn + 16 * jc, LDB, lane);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * bt + 4 * lg + r;
        sdU[row * LDF + 16 * jc + lr] = acc[r] + vec[V_KF * C + row] * acc2[r];
      }
    }
    lds_barrier();
    // -- dZ = (I + A)^-T dU by blocks, last block first, one wavefront per column tile;
    //    the other wavefronts stage the next chunk meanwhile
    if (wave < NJ) {
      const int jc = wave;
#pragma unroll
      for (int b = 3; b >= 0; --b) {
        floatx4 w, sub = zero4();
#pragma unroll
        for (int r = 0; r < 4; ++r) w[r] = sdU[(16 * b + 4 * lg + r) * LDF + 16 * jc + lr];
        for (int m = b + 1; m < 4; ++m)
          tile_mm<T, true, true, 16>(sub, sA + 16 * m * LDC + 16 * b, LDC, sdZ + 16 * m * LDB + 16 * jc, LDB, lane);
        w -= sub;
        floatx4 u = zero4();
        Mma16<T>::mma(u, lds_col4<T>(sTd + b * 16 * LDD, LDD, 0, 0, lane), Mma16<T>::chain(w));
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * b + 4 * lg + r;
          const T zt = from_float<T>(u[r]);
          const float bt = vec[V_BETA * C + row];
          sdZ[row * LDB + 16 * jc + lr] = zt;
          sdZb[row * LDB + 16 * jc + lr] = from_float<T>(-bt * vec[V_GAM * C + row] * u[r]);
          sdU[row * LDF + 16 * jc + lr] = u[r];  // (this block's dU is read) dZ, for the copy-out
        }
      }
    } else if (c > 0) {
      if constexpr (AHEAD) {
        stage_store(c - 1);
        if (c > 1) stage_load(c - 2);
      } else {
        stage_in(c - 1, 64 * NJ, std::integral_constant<int, NST>());
      }
    }
    lds_barrier();
    // -- dZ (workspace, T) and dv = beta dZ out as whole 16-byte pieces, by every
    //    wavefront (the solving ones only wrote LDS)
    if (tid < C * BV / 4) {
      const int row = tid / (BV / 4), c4 = (tid - row * (BV / 4)) * 4;
      if (row < Lc) {
        const floatx4 z = *reinterpret_cast<const floatx4*>(sdU + row * LDF + c4);
        const float bt = vec[V_BETA * C + row];
        const size_t o0 = (static_cast<size_t>(cs + row) * p.Hv + h) * DV + col0 + c4;
        *reinterpret_cast<floatx4*>(p.dv + o0) = bt * z;
        *reinterpret_cast<typename Vec4<T>::type*>(static_cast<T*>(p.dz) + o0) = pack4<T>(z[0], z[1], z[2], z[3]);
      }
    }
    // -- dM = gam_C dM' + s Q^T diag(gam) dO - K^T diag(beta gam) dZ, then its operand copy
    {
      const float gC = vec[V_N * C];
      static_assert(NW % NJ == 0, "a wavefront's tiles share one column block");
      const int jc = wave % NJ;
      const ColFrags<T, C> og(sdOg + 16 * jc, LDB, lane), zb(sdZb + 16 * jc, LDB, lane);
#pragma unroll
      for (int i = 0; i < NMT; ++i) {
        const int t = wave + NW * i, a = t / NJ;
        if (t >= NTL) break;
        dM[i] *= gC;
        tile_mm<T, true, C>(dM[i], sQ + 16 * a, LDK, og, lane);
        tile_mm<T, true, C>(dM[i], sK + 16 * a, LDK, zb, lane);
      }
      dm_to_lds();  // (dU, the only reader, is done: the barrier above)
    }
    lds_barrier();
  }
  if (p.dh0) {
#pragma unroll
    for (int i = 0; i < NMT; ++i) {
      const int t = wave + NW * i, a = t / NJ, jc = t % NJ;
      if (t >= NTL) break;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        p.dh0[sbase + static_cast<size_t>(16 * a + 4 * lg + r) * DV + col0 + 16 * jc + lr] = dM[i][r];
    }
  }
}

// ------------------------------------------------------- per-chunk gradients
template <class T, int DK, int DV>
struct DlLayout {
  static constexpr int PAD = 32 / sizeof(T);
  static constexpr int LDK = DK + PAD, LDV = DV + PAD, LDC = C + PAD / 2;
  static constexpr int KTL = DK / 16;             // key-dim tiles (16-column blocks of dq and dk)
  static constexpr int NOT = (C / 16) * KTL / 8;  // dq (and dk) tiles per wavefront
  static constexpr int oQ = 0;
  static constexpr int oK = oQ + C * LDK * sizeof(T);
  static constexpr int odO = oK + C * LDK * sizeof(T);
  static constexpr int oU = odO + C * LDV * sizeof(T);
  static constexpr int odZ = oU + C * LDV * sizeof(T);
  static constexpr int oM = odZ + C * LDV * sizeof(T);  // M, then dM'
  static constexpr int odP = oM + DK * LDV * sizeof(T);
  static constexpr int oS = odP + C * LDC * sizeof(T);
  static constexpr int oVec = oS + C * LDC * sizeof(T);
  // The per-token sums that make dG and dbeta, one slot per contribution, each
  // written once per value head and added in a fixed order at the end (so the
  // gradients do not depend on the order in which wavefronts finish):
  //   RG [kind][tj][token]  row sums of the Gram tiles (kind 0: dP, 1: dA) of column block tj
  //   CG [kind][ti][token]  their column sums, by row block ti
  //   RB [tj][token]        the dbeta row sums of the dA tiles
  //   B0 [token]            the dZ . v part of dbeta
  //   QG, QB [kt][token]    the dq / dk tiles' terms of key block kt (dG, dbeta)
  //   DG [kt][token]        the U dM'^T tiles' terms
  //   SC                    terms of the last token: <dM', M> per wavefront, then
  //                         the U dM'^T terms per wavefront and tile
  static constexpr int oRG = oVec + (V_N * C + 4) * 4;
  static constexpr int oCG = oRG + 2 * 4 * C * 4;
  static constexpr int oRB = oCG + 2 * 4 * C * 4;
  static constexpr int oB0 = oRB + 4 * C * 4;
  static constexpr int oQG = oB0 + C * 4;
  static constexpr int oQB = oQG + KTL * C * 4;
  static constexpr int oDG = oQB + KTL * C * 4;
  static constexpr int oSC = oDG + KTL * C * 4;
  static constexpr int bytes = oSC + (8 + 8 * NOT) * 4;
};

// One workgroup per (chunk, query/key head): it walks the value heads that
// share the query/key head, summing their dq and dk tiles in registers, and
// writes every gradient element once with a plain store.
template <class T, int DK, int DV>
__global__ __launch_bounds__(512) void dlocal_kernel(BwdParams p) {
  using L = DlLayout<T, DK, DV>;
  constexpr int LDK = L::LDK, LDV = L::LDV, LDC = L::LDC, NT = 512;
  constexpr int KTL = L::KTL, NOT = L::NOT;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  T* sQ = reinterpret_cast<T*>(smem + L::oQ);
  T* sK = reinterpret_cast<T*>(smem + L::oK);
  T* sdO = reinterpret_cast<T*>(smem + L::odO);
  T* sU = reinterpret_cast<T*>(smem + L::oU);
  T* sdZ = reinterpret_cast<T*>(smem + L::odZ);
  T* sM = reinterpret_cast<T*>(smem + L::oM);
  T* sdP = reinterpret_cast<T*>(smem + L::odP);
  T* sS = reinterpret_cast<T*>(smem + L::oS);
  float* vec = reinterpret_cast<float*>(smem + L::oVec);
  float* sRG = reinterpret_cast<float*>(smem + L::oRG);
  float* sCG = reinterpret_cast<float*>(smem + L::oCG);
  float* sRB = reinterpret_cast<float*>(smem + L::oRB);
  float* sB0 = reinterpret_cast<float*>(smem + L::oB0);
  float* sQG = reinterpret_cast<float*>(smem + L::oQG);
  float* sQB = reinterpret_cast<float*>(smem + L::oQB);
  float* sDG = reinterpret_cast<float*>(smem + L::oDG);
  float* sSC = reinterpret_cast<float*>(smem + L::oSC);

  const int tid0 = threadIdx.x;
  const int gc = blockIdx.x / p.Hqk, hq = blockIdx.x - (blockIdx.x / p.Hqk) * p.Hqk;
  // the chunk's sequence: the last n with chunk base <= gc
  int n, c;
  if (p.cu) {
    if (gc >= p.cpre[p.N]) return;
    int lo = 0, hi = p.N;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (p.cpre[mid] <= gc) lo = mid; else hi = mid;
    }
    n = lo;
    c = gc - p.cpre[n];
  } else {
    const int per = (p.T + C - 1) / C;
    if (per == 0) return;
    n = gc / per;
    c = gc - n * per;
    if (n >= p.N) return;
  }
  const Seq sq = seq_of(p.cu, p.cpre, p.T, n);
  const int cs = sq.bos + c * C, Lc = min(C, sq.eos - cs);
  const int rep = p.Hv / p.Hqk;
  const size_t qk_tok = static_cast<size_t>(p.Hqk) * DK, v_tok = static_cast<size_t>(p.Hv) * DV;
  const float s = p.scale;
  const size_t qo = static_cast<size_t>(cs) * qk_tok + static_cast<size_t>(hq) * DK;
  // A wavefront's dq and dk tiles share one 16-column block kt (tile t = wave + 8i, kt = t % KTL), so
  // the B operands are read once for all of them.
  static_assert(8 % KTL == 0, "one key block per wavefront");
  floatx4 dqa[NOT], dka[NOT];  // dq and dk tiles, summed over the value heads
#pragma unroll
  for (int i = 0; i < NOT; ++i) dqa[i] = dka[i] = zero4();

  for (int hh = 0; hh < rep; ++hh) {
    // The body's LDS addresses derive from the thread index; formed from an
    // opaque copy of it each pass, they are computed where they are used
    // rather than hoisted out of the loop and held in registers throughout.
    int tid;
    asm volatile("v_mov_b32 %0, %1" : "=v"(tid) : "v"(tid0));
    const int lane = tid & 63, wave = tid >> 6, lg = lane >> 4, lr = lane & 15, kt = wave % KTL;
    const int h = hq * rep + hh;
    const size_t ck = (static_cast<size_t>(sq.cbase + c) * p.Hv + h) * DK * DV;
    const size_t vo = static_cast<size_t>(cs) * v_tok + static_cast<size_t>(h) * DV;
    // -- stage: Q and K (once), dO, U, dZ, M; gates.  Every global operand is requested first, so the
    //    workgroup waits for memory once per value head; v and dM' stay in registers until they are used.
    RowsInFlight<T, DV, NT> rv;
    RowsInFlight<T, DV, NT, DK> rdm;
    {
      RowsInFlight<T, DK, NT> rq, rk;
      RowsInFlight<T, DV, NT> rdo, ru, rdz;
      RowsInFlight<T, DV, NT, DK> rm;
      if (hh == 0) {
        rq.load(static_cast<const T*>(p.q) + qo, qk_tok, Lc, tid);
        rk.load(static_cast<const T*>(p.k) + qo, qk_tok, Lc, tid);
      }
      rdo.load(static_cast<const T*>(p.dout) + vo, v_tok, Lc, tid);
      ru.load(static_cast<const T*>(p.ck_u) + vo, v_tok, Lc, tid);
      rdz.load(static_cast<const T*>(p.dz) + vo, v_tok, Lc, tid);
      rm.load(static_cast<const T*>(p.ck_state) + ck, DV, DK, tid);
      rv.load(static_cast<const T*>(p.v) + vo, v_tok, Lc, tid);
      rdm.load(static_cast<const T*>(p.dm) + ck, DV, DK, tid);
      float gt = 0.f, bt = 0.f;  // tokens past the end act as g = 0, beta = 0
      if (wave == 0 && lane < Lc) {
        const size_t gi = static_cast<size_t>(cs + lane) * p.Hv + h;
        gt = p.g[gi];
        bt = p.beta[gi];
      }
      if (hh > 0) lds_barrier();  // the previous value head's reads of LDS are done
      if (wave == 0) gate_vectors_from(vec, gt, bt, lane);
      if (hh == 0) {
        rq.store(sQ, LDK, tid);
        rk.store(sK, LDK, tid);
      }
      rdo.store(sdO, LDV, tid);
      ru.store(sU, LDV, tid);
      rdz.store(sdZ, LDV, tid);
      rm.store(sM, LDV, tid);
    }
    lds_barrier();
    {  // the dZ . v part of dbeta
      constexpr int EP = decltype(rv)::EP, PR = DV / EP, IT = C * PR / NT;
      static_assert(C * PR % NT == 0 && NT % PR == 0 && IT == decltype(rv)::IT, "whole rows per pass");
      static_assert(PR == 8 || PR == 16 || PR == 32, "a row is half, one or two 16-lane groups");
#pragma unroll
      for (int it = 0; it < IT; ++it) {
        const int i = tid + it * NT, t = i / PR, e = (i - t * PR) * EP;
        float part = 0.f;
#pragma unroll
        for (int x = 0; x < EP; ++x) part += to_float(sdZ[t * LDV + e + x]) * to_float(rv.v[it][x]);
        if constexpr (PR == 8) part = sum8(part);  // the row's lanes first
        else part = sum16(part);
        if constexpr (PR == 32) part += __shfl_xor(part, 16);
        if ((lane & (PR - 1)) == 0) sB0[t] = part;
      }
    }
    // -- C x C tiles: dP (masked, times s exp(G_i - G_j)) and D + D^T, with their dG and dbeta terms
    for (int job = wave; job < 20; job += 8) {
      const int kind = job / 10, lt = job % 10;
      const int ti = lt < 1 ? 0 : lt < 3 ? 1 : lt < 6 ? 2 : 3;
      const int tj = lt - ti * (ti + 1) / 2;
      floatx4 gr = zero4(), d = zero4();
      tile_mm_nn<T, DK>(gr, (kind ? sK : sQ) + 16 * ti * LDK, LDK, sK + 16 * tj * LDK, LDK, lane);
      tile_mm_nn<T, DV>(d, (kind ? sdZ : sdO) + 16 * ti * LDV, LDV, sU + 16 * tj * LDV, LDV, lane);
      const int j = 16 * tj + lr, i0 = 16 * ti + 4 * lg;
      const floatx4 Gi = vec4_at(vec + V_GL * C + i0), bi = vec4_at(vec + V_BETA * C + i0);
      const float Gj = vec[V_GL * C + j];
      float colsum = 0.f;
      floatx4 rw, rb;
#pragma unroll
      for (int r = 0; r < 4; ++r) {  // branch-free: the masks are selects
        const int i = i0 + r;
        const float e = __builtin_amdgcn_exp2f(Gi[r] - Gj);
        float w, rowb = 0.f;
        if (kind == 0) {  // P_ij = s dec (QK^T)_ij, dP_ij = (dO U^T)_ij, j <= i
          const float dps = j <= i ? d[r] * s * e : 0.f;  // dP s dec
          w = dps * gr[r];
          sdP[i * LDC + j] = from_float<T>(dps);
        } else {  // A_ij = beta_i dec (KK^T)_ij, dA_ij = -(dZ U^T)_ij, j < i
          const float dae = j < i ? -d[r] * e : 0.f;  // dA dec
          w = dae * bi[r] * gr[r];
          rowb = dae * gr[r];
          const T dd = from_float<T>(dae * bi[r]);
          if (j < i) sS[j * LDC + i] = dd;
          if (j <= i) sS[i * LDC + j] = dd;  // (zero on the diagonal)
        }
        colsum += w;
        rw[r] = sum16(w);
        rb[r] = sum16(rowb);
      }
      if (kind == 0 && ti != tj) {  // the tile above the diagonal is zero
#pragma unroll
        for (int r = 0; r < 4; ++r) sdP[j * LDC + i0 + r] = from_float<T>(0.f);
      }
      if (lr == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          sRG[(kind * 4 + tj) * C + i0 + r] = rw[r];
          if (kind) sRB[tj * C + i0 + r] = rb[r];
        }
      }
      colsum += __shfl_xor(colsum, 16);
      colsum += __shfl_xor(colsum, 32);
      if (lg == 0) sCG[(kind * 4 + ti) * C + j] = -colsum;
    }
    lds_barrier();
    // -- dq += s diag(gam) dO M^T + (dP s dec) K;
    //    dk += -diag(beta gam) dZ M^T + (dP s dec)^T Q + (D + D^T) K  (the dM' term follows)
    {
      const RowFrags<T, DV> mf(sM + 16 * kt * LDV, LDV, lane);  // M rows of the block
      const ColFrags<T, C> kcol(sK + 16 * kt, LDK, lane), qcol(sQ + 16 * kt, LDK, lane);
#pragma unroll
      for (int i = 0; i < NOT; ++i) {
        const int t = wave + 8 * i, it = t / KTL;
        floatx4 a = zero4(), b = zero4();
        tile_mm_nn<T, DV>(a, sdO + 16 * it * LDV, LDV, mf, lane);  // dO M^T
        tile_mm_nn<T, DV>(b, sdZ + 16 * it * LDV, LDV, mf, lane);  // dZ M^T
        {
          const int r0 = 16 * it + 4 * lg, key = 16 * kt + lr;
          const floatx4 gam = vec4_at(vec + V_GAM * C + r0), bt = vec4_at(vec + V_BETA * C + r0);
          floatx4 gq, gk;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            dqa[i][r] += s * gam[r] * a[r];
            dka[i][r] -= bt[r] * gam[r] * b[r];
            gq[r] = sum16(to_float(sQ[(r0 + r) * LDK + key]) * a[r]);
            gk[r] = sum16(to_float(sK[(r0 + r) * LDK + key]) * b[r]);
          }
          if (lr == 0) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              sQG[kt * C + r0 + r] = s * gam[r] * gq[r] - bt[r] * gam[r] * gk[r];
              sQB[kt * C + r0 + r] = -gam[r] * gk[r];
            }
          }
        }
        tile_mm<T, false, C>(dqa[i], sdP + 16 * it * LDC, LDC, kcol, lane);
        tile_mm<T, true, C>(dka[i], sdP + 16 * it, LDC, qcol, lane);
        tile_mm<T, false, C>(dka[i], sS + 16 * it * LDC, LDC, kcol, lane);
      }
    }
    // -- dM' replaces M in LDS; gam_C <dM', M> enters dG at the chunk's end
    {
      constexpr int EP = decltype(rdm)::EP, PR = DV / EP, IT = DK * PR / NT;
      static_assert(DK * PR % NT == 0 && IT == decltype(rdm)::IT, "whole passes");
      float part = 0.f;
#pragma unroll
      for (int it = 0; it < IT; ++it) {
        const int i = tid + it * NT, r = i / PR, e = (i - r * PR) * EP;
#pragma unroll
        for (int x = 0; x < EP; ++x) part += to_float(rdm.v[it][x]) * to_float(sM[r * LDV + e + x]);
      }
      part = sum16(part);
      part += __shfl_xor(part, 16);
      part += __shfl_xor(part, 32);
      if (lane == 0) sSC[wave] = vec[V_N * C] * part;
      lds_barrier();  // every M value is read before dM' replaces it
      rdm.store(sM, LDV, tid);
    }
    lds_barrier();
    // -- dk += diag(kf) U dM'^T, with its dG terms
    {
      const RowFrags<T, DV> dmf(sM + 16 * kt * LDV, LDV, lane);  // dM' rows of the block
#pragma unroll
      for (int i = 0; i < NOT; ++i) {
        const int t = wave + 8 * i, it = t / KTL;
        floatx4 a = zero4();
        tile_mm_nn<T, DV>(a, sU + 16 * it * LDV, LDV, dmf, lane);  // U dM'^T
        const int r0 = 16 * it + 4 * lg, key = 16 * kt + lr;
        const floatx4 kf = vec4_at(vec + V_KF * C + r0);
        floatx4 sj;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          dka[i][r] += kf[r] * a[r];
          sj[r] = kf[r] * sum16(to_float(sK[(r0 + r) * LDK + key]) * a[r]);
        }
        if (lr == 0) {
#pragma unroll
          for (int r = 0; r < 4; ++r) sDG[kt * C + r0 + r] = -sj[r];
        }
        float tot = (sj[0] + sj[1]) + (sj[2] + sj[3]);  // this tile's part of the last token's term
        tot += __shfl_xor(tot, 16);
        tot += __shfl_xor(tot, 32);
        if (lane == 0) sSC[8 + wave * NOT + i] = tot;
      }
    }
    lds_barrier();
    // -- dg = reverse cumsum of dG over the chunk; dbeta.  The slots of token t, added in a fixed order.
    if (wave == 0) {
      const int t = C - 1 - lane, tt = t / 16;
      float dG = 0.f, dB = sB0[t];
#pragma unroll
      for (int kind = 0; kind < 2; ++kind)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          if (b <= tt) dG += sRG[(kind * 4 + b) * C + t];  // tiles (tt, b), b <= tt
          if (b >= tt) dG += sCG[(kind * 4 + b) * C + t];  // tiles (b, tt), b >= tt
        }
#pragma unroll
      for (int b = 0; b < 4; ++b)
        if (b <= tt) dB += sRB[b * C + t];
#pragma unroll
      for (int x = 0; x < KTL; ++x) {
        dG += sQG[x * C + t] + sDG[x * C + t];
        dB += sQB[x * C + t];
      }
      if (t == C - 1) {
#pragma unroll
        for (int x = 0; x < 8 + 8 * NOT; ++x) dG += sSC[x];
      }
      const float dg = wave_inclusive_sum(dG);
      if (t < Lc) {
        const size_t gi = static_cast<size_t>(cs + t) * p.Hv + h;
        p.dg[gi] = dg;
        p.dbeta[gi] = dB;
      }
    }
  }
  // -- dq and dk, the sums over the value heads
  const int lane = tid0 & 63, wave = tid0 >> 6, lg = lane >> 4, lr = lane & 15, kt = wave % KTL;
#pragma unroll
  for (int i = 0; i < NOT; ++i) {
    const int it = (wave + 8 * i) / KTL;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 16 * it + 4 * lg + r;
      if (row < Lc) {
        const size_t o = qo + static_cast<size_t>(row) * qk_tok + 16 * kt + lr;
        p.dq[o] = dqa[i][r];
        p.dk[o] = dka[i][r];
      }
    }
  }
}

// Exclusive prefix sum of the chunk counts of the packed sequences: out[n] is
// the global index of sequence n's first chunk, out[N] the total.
__global__ __launch_bounds__(1024) void chunk_prefix_kernel(const int32_t* cu, int N, int32_t* out) {
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

template <class T, int DK, int DV, int BV>
hipError_t launch(const BwdArgs& a, hipStream_t stream) {
  using LS = DsLayout<T, DK, BV>;
  using LL = DlLayout<T, DK, DV>;
  static_assert(LS::bytes <= 160 * 1024 && LL::bytes <= 160 * 1024, "LDS budget of one gfx950 compute unit");
  const int64_t tokens = static_cast<int64_t>(a.batch) * a.seqlen;
  const BwdParts w = bwd_parts(tokens, a.num_seqs, a.Hv, DK, DV, sizeof(T) == 2);
  unsigned char* ws = static_cast<unsigned char*>(a.workspace);  // 256-byte aligned
  int32_t* cpre = a.cu_seqlens ? reinterpret_cast<int32_t*>(ws + w.cpre) : nullptr;
  if (cpre) chunk_prefix_kernel<<<dim3(1), dim3(1024), 0, stream>>>(a.cu_seqlens, a.num_seqs, cpre);

  PrefillArgs f;
  f.q = a.q;
  f.k = a.k;
  f.v = a.v;
  f.g = a.g;
  f.beta = a.beta;
  f.initial_state = a.initial_state;
  f.cu_seqlens = a.cu_seqlens;
  f.o = nullptr;
  f.final_state = nullptr;
  f.batch = a.batch;
  f.seqlen = a.seqlen;
  f.num_seqs = a.num_seqs;
  f.Hqk = a.Hqk;
  f.Hv = a.Hv;
  f.dk = DK;
  f.dv = DV;
  f.chunk = C;
  f.scale = a.scale;
  f.bf16 = sizeof(T) == 2;
  f.save_state = ws + w.state;
  f.save_u = ws + w.u;
  f.chunk_base = cpre;
  hipError_t e = launch_prefill(f, stream);
  if (e != hipSuccess) return e;

  BwdParams p;
  p.q = a.q;
  p.k = a.k;
  p.v = a.v;
  p.dout = a.dout;
  p.g = a.g;
  p.beta = a.beta;
  p.dhT = a.d_final_state;
  p.cu = a.cu_seqlens;
  p.cpre = cpre;
  p.ck_state = f.save_state;
  p.ck_u = f.save_u;
  p.dm = ws + w.dm;
  p.dz = ws + w.dz;
  p.dq = a.dq;
  p.dk = a.dk;
  p.dv = a.dv;
  p.dg = a.dg;
  p.dbeta = a.dbeta;
  p.dh0 = a.d_initial_state;
  p.T = a.seqlen;
  p.N = a.num_seqs;
  p.Hqk = a.Hqk;
  p.Hv = a.Hv;
  p.chunk_bound = static_cast<int>(tokens / C + a.num_seqs);
  p.scale = a.scale;
  const int units = a.num_seqs * a.Hv;
  if (units == 0) return hipGetLastError();
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(&dstate_kernel<T, DK, DV, BV>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, LS::bytes);
  if (e != hipSuccess) return e;
  dstate_kernel<T, DK, DV, BV><<<dim3((units + 7) / 8 * 8 * (DV / BV)), dim3(512), LS::bytes, stream>>>(p);
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(&dlocal_kernel<T, DK, DV>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, LL::bytes);
  if (e != hipSuccess) return e;
  dlocal_kernel<T, DK, DV><<<dim3(p.chunk_bound * a.Hqk), dim3(512), LL::bytes, stream>>>(p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream) {
  if (a.bf16) {
    if (a.head_dim_k == 128 && a.head_dim_v == 128) return launch<bf16, 128, 128, 32>(a, stream);
    if (a.head_dim_k == 64 && a.head_dim_v == 64) return launch<bf16, 64, 64, 32>(a, stream);
  } else {
    if (a.head_dim_k == 64 && a.head_dim_v == 64) return launch<float, 64, 64, 16>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdn

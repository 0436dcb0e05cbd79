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
//      state and U (fp32 workspace);
//   2. dstate_kernel walks each (sequence, value head, 32-column slice of dv)
//      backwards over its chunks, holding dM in registers: it keeps dM' and dZ
//      per chunk and leaves dM of the first chunk as the initial state's gradient;
//   3. dlocal_kernel forms every per-token gradient of one chunk and one
//      query/key head (looping over the value heads that share it, so dq and
//      dk are summed without atomics), all chunks in parallel.
// Products run on the matrix cores over 16-wide k-steps with operands in LDS
// (bf16 inputs: bf16 operands, fp32 accumulation; fp32 inputs: fp32 throughout).
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
template <class T, bool TA, bool TB>
__device__ __forceinline__ void tile_mm(floatx4& acc, const T* A, int lda, const T* B, int ldb, int K, int lane) {
  for (int k0 = 0; k0 < K; k0 += 16) {
    const auto fa = TA ? lds_col4<T>(A + k0 * lda, lda, 0, 0, lane) : row4<T>(A + k0, lda, lane);
    const auto fb = TB ? lds_col4<T>(B + k0 * ldb, ldb, 0, 0, lane) : row4<T>(B + k0, ldb, lane);
    Mma16<T>::mma(acc, fa, fb);
  }
}

__device__ __forceinline__ float sum16(float x) {  // over the 16 lanes of a row group
  x += __shfl_xor(x, 1);
  x += __shfl_xor(x, 2);
  x += __shfl_xor(x, 4);
  x += __shfl_xor(x, 8);
  return x;
}
__device__ __forceinline__ float rdlane(float x, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
}

__device__ __forceinline__ floatx4 load4(const float* p) { return *reinterpret_cast<const floatx4*>(p); }
__device__ __forceinline__ floatx4 load4(const bf16* p) {
  const bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
  return floatx4{to_float(v[0]), to_float(v[1]), to_float(v[2]), to_float(v[3])};
}
template <class D>
__device__ __forceinline__ void store4(D* p, const floatx4& v) {
  *reinterpret_cast<typename Vec4<D>::type*>(p) = pack4<D>(v[0], v[1], v[2], v[3]);
}

// Rows [0, C) of W columns from a token-major source (row stride ss elements)
// into an LDS tile (row stride ld); rows >= L are zero.
template <class S, class D, int W>
__device__ __forceinline__ void stage_rows(D* dst, int ld, const S* src, size_t ss, int L, int tid, int nt) {
  constexpr int PR = W / 4;
  for (int i = tid; i < C * PR; i += nt) {
    const int t = i / PR, e = (i - t * PR) * 4;
    const floatx4 v = t < L ? load4(src + t * ss + e) : zero4();
    store4<D>(dst + t * ld + e, v);
  }
}

// Per-chunk gate vectors, formed by one wavefront (lane = token): log2-scaled
// inclusive cumsum Gl, exp(G), exp(G_C - G), beta (tokens >= L act as g = 0,
// beta = 0), and exp(G_C) in vec[4C].
enum { V_GL, V_GAM, V_KF, V_BETA, V_N };
__device__ __forceinline__ void gate_vectors(float* vec, const float* g, const float* beta, size_t stride, int L,
                                             int lane) {
  const bool live = lane < L;
  const float gt = live ? g[lane * stride] : 0.f;
  const float bt = live ? beta[lane * stride] : 0.f;
  const float Gl = wave_inclusive_sum(gt) * kLog2e;
  const float GlC = rdlane(Gl, 63);
  vec[V_GL * C + lane] = Gl;
  vec[V_GAM * C + lane] = __builtin_amdgcn_exp2f(Gl);
  vec[V_KF * C + lane] = __builtin_amdgcn_exp2f(GlC - Gl);
  vec[V_BETA * C + lane] = bt;
  if (lane == 0) vec[V_N * C] = __builtin_amdgcn_exp2f(GlC);
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
  const float *ck_state, *ck_u;  // chunk-start states, U (from the saving prefill)
  float *dm, *dz;                // dM' per chunk, dZ per token (dstate_kernel)
  float *dq, *dk, *dv, *dg, *dbeta, *dh0;
  int T, N, Hqk, Hv, chunk_bound;
  float scale;
};

// ------------------------------------------------------- state gradient scan
template <class T, int DK, int BV>
struct DsLayout {
  static constexpr int PAD = 32 / sizeof(T);  // 32-byte row padding
  static constexpr int LDK = DK + PAD, LDB = BV + PAD, LDC = C + PAD, LDD = 16 + PAD, LDF = BV + 4, LDT = 20;
  static constexpr int oK = 0;
  static constexpr int oQ = oK + C * LDK * sizeof(T);
  static constexpr int odO = oQ + C * LDK * sizeof(T);
  static constexpr int odOg = odO + C * LDB * sizeof(T);  // s gam dO
  static constexpr int odZ = odOg + C * LDB * sizeof(T);
  static constexpr int odZb = odZ + C * LDB * sizeof(T);  // -beta gam dZ
  static constexpr int odMn = odZb + C * LDB * sizeof(T);
  static constexpr int oP = odMn + DK * LDB * sizeof(T);
  static constexpr int oA = oP + C * LDC * sizeof(T);
  static constexpr int oTd = oA + C * LDC * sizeof(T);  // diagonal blocks of (I + A)^-1, row-major
  static constexpr int odU = oTd + 4 * 16 * LDD * sizeof(T);  // fp32
  static constexpr int oAt = odU + C * LDF * 4;               // fp32 diagonal blocks of A, transposed
  static constexpr int oVec = oAt + 4 * 16 * LDT * 4;
  static constexpr int bytes = oVec + (V_N * C + 4) * 4;
};

template <class T, int DK, int DV, int BV>
__global__ __launch_bounds__(256) void dstate_kernel(BwdParams p) {
  using L = DsLayout<T, DK, BV>;
  constexpr int LDK = L::LDK, LDB = L::LDB, LDC = L::LDC, LDD = L::LDD, LDF = L::LDF, LDT = L::LDT;
  constexpr int NJ = BV / 16;              // column tiles of the slice
  constexpr int NMT = (DK / 16) * NJ / 4;  // dM tiles per wavefront
  static_assert((DK / 16) * NJ % 4 == 0 && 4 * NJ % 4 == 0, "tiles split over four wavefronts");
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  T* sK = reinterpret_cast<T*>(smem + L::oK);
  T* sQ = reinterpret_cast<T*>(smem + L::oQ);
  T* sdO = reinterpret_cast<T*>(smem + L::odO);
  T* sdOg = reinterpret_cast<T*>(smem + L::odOg);
  T* sdZ = reinterpret_cast<T*>(smem + L::odZ);
  T* sdZb = reinterpret_cast<T*>(smem + L::odZb);
  T* sdMn = reinterpret_cast<T*>(smem + L::odMn);
  T* sP = reinterpret_cast<T*>(smem + L::oP);
  T* sA = reinterpret_cast<T*>(smem + L::oA);
  T* sTd = reinterpret_cast<T*>(smem + L::oTd);
  float* sdU = reinterpret_cast<float*>(smem + L::odU);
  float* sAt = reinterpret_cast<float*>(smem + L::oAt);
  float* vec = reinterpret_cast<float*>(smem + L::oVec);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lg = lane >> 4, lr = lane & 15;
  constexpr int NS = DV / BV;
  const int unit = blockIdx.x / NS;
  const int col0 = (blockIdx.x - unit * NS) * BV;
  const int n = unit / p.Hv, h = unit - n * p.Hv, hq = h / (p.Hv / p.Hqk);
  const Seq sq = seq_of(p.cu, p.cpre, p.T, n);
  const int nch = (sq.eos - sq.bos + C - 1) / C;
  const size_t sbase = static_cast<size_t>(unit) * DK * DV;
  const T* qg = static_cast<const T*>(p.q);
  const T* kg = static_cast<const T*>(p.k);
  const T* dog = static_cast<const T*>(p.dout);
  const size_t qk_tok = static_cast<size_t>(p.Hqk) * DK, v_tok = static_cast<size_t>(p.Hv) * DV;

  // dM tiles of this wavefront: tile t = wave + 4i -> rows 16 (t / NJ), columns 16 (t % NJ)
  floatx4 dM[NMT];
#pragma unroll
  for (int i = 0; i < NMT; ++i) {
    const int t = wave + 4 * i, a = t / NJ, jc = t % NJ;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      dM[i][r] = p.dhT ? p.dhT[sbase + static_cast<size_t>(16 * a + 4 * lg + r) * DV + col0 + 16 * jc + lr] : 0.f;
  }

  for (int c = nch - 1; c >= 0; --c) {
    const int cs = sq.bos + c * C, Lc = min(C, sq.eos - cs);
    // -- stage: K, Q, dO slice, gates; dM' to LDS (operands) and to the workspace
    stage_rows<T, T, DK>(sK, LDK, kg + static_cast<size_t>(cs) * qk_tok + static_cast<size_t>(hq) * DK, qk_tok, Lc,
                         tid, 256);
    stage_rows<T, T, DK>(sQ, LDK, qg + static_cast<size_t>(cs) * qk_tok + static_cast<size_t>(hq) * DK, qk_tok, Lc,
                         tid, 256);
    stage_rows<T, T, BV>(sdO, LDB, dog + static_cast<size_t>(cs) * v_tok + static_cast<size_t>(h) * DV + col0, v_tok,
                         Lc, tid, 256);
    if (wave == 0) {
      const size_t gi = static_cast<size_t>(cs) * p.Hv + h;
      gate_vectors(vec, p.g + gi, p.beta + gi, p.Hv, Lc, lane);
    }
    {
      float* dmw = p.dm + (static_cast<size_t>(sq.cbase + c) * p.Hv + h) * DK * DV;
#pragma unroll
      for (int i = 0; i < NMT; ++i) {
        const int t = wave + 4 * i, a = t / NJ, jc = t % NJ;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * a + 4 * lg + r, col = 16 * jc + lr;
          sdMn[row * LDB + col] = from_float<T>(dM[i][r]);
          dmw[static_cast<size_t>(row) * DV + col0 + col] = dM[i][r];
        }
      }
    }
    __syncthreads();
    // -- Gram tiles: P and A (lower tiles), s gam dO
    {
      const float s = p.scale;
      for (int job = wave; job < 20; job += 4) {
        const int kind = job / 10, lt = job % 10;  // lower tile lt -> (ti, tj)
        const int ti = lt < 1 ? 0 : lt < 3 ? 1 : lt < 6 ? 2 : 3;
        const int tj = lt - ti * (ti + 1) / 2;
        floatx4 acc = zero4();
        tile_mm<T, false, false>(acc, (kind ? sK : sQ) + 16 * ti * LDK, LDK, sK + 16 * tj * LDK, LDK, DK, lane);
        const int j = 16 * tj + lr;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 16 * ti + 4 * lg + r;
          const float dec = j <= i ? __builtin_amdgcn_exp2f(vec[V_GL * C + i] - vec[V_GL * C + j]) : 0.f;
          if (kind == 0) {
            sP[i * LDC + j] = from_float<T>(s * dec * acc[r]);
          } else {
            const float a = j < i ? vec[V_BETA * C + i] * dec * acc[r] : 0.f;
            sA[i * LDC + j] = from_float<T>(a);
            if (ti == tj) sAt[(ti * 16 + (j & 15)) * LDT + (i & 15)] = a;
          }
        }
      }
      for (int i = tid; i < C * BV; i += 256) {
        const int t = i / BV, cc = i - t * BV;
        sdOg[t * LDB + cc] = from_float<T>(s * vec[V_GAM * C + t] * to_float(sdO[t * LDB + cc]));
      }
    }
    __syncthreads();
    // -- inverses of the diagonal blocks of I + A; dU = P^T dO + diag(kf) K dM'
    {
      const int cc = lane >> 2, q = lane & 3;
      floatx4 x;
#pragma unroll
      for (int t = 0; t < 4; ++t) x[t] = (4 * q + t == cc) ? 1.f : 0.f;
      unit_lower_inverse_column(x, sAt + wave * 16 * LDT, LDT, q, std::make_integer_sequence<int, 15>());
#pragma unroll
      for (int t = 0; t < 4; ++t) sTd[(wave * 16 + 4 * q + t) * LDD + cc] = from_float<T>(x[t]);
    }
    for (int t = wave; t < 4 * NJ; t += 4) {
      const int bt = t / NJ, jc = t % NJ;
      floatx4 acc = zero4(), acc2 = zero4();
      tile_mm<T, true, true>(acc, sP + 16 * bt * LDC + 16 * bt, LDC, sdO + 16 * bt * LDB + 16 * jc, LDB, C - 16 * bt,
                             lane);
      tile_mm<T, false, true>(acc2, sK + 16 * bt * LDK, LDK, sdMn + 16 * jc, LDB, DK, lane);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * bt + 4 * lg + r;
        sdU[row * LDF + 16 * jc + lr] = acc[r] + vec[V_KF * C + row] * acc2[r];
      }
    }
    __syncthreads();
    // -- dZ = (I + A)^-T dU by blocks, last block first; one wavefront per column tile
    if (wave < NJ) {
      const int jc = wave;
      float* dzw = p.dz + (static_cast<size_t>(cs) * p.Hv + h) * DV + col0 + 16 * jc + lr;
#pragma unroll
      for (int b = 3; b >= 0; --b) {
        floatx4 w, sub = zero4();
#pragma unroll
        for (int r = 0; r < 4; ++r) w[r] = sdU[(16 * b + 4 * lg + r) * LDF + 16 * jc + lr];
        for (int m = b + 1; m < 4; ++m)
          tile_mm<T, true, true>(sub, sA + 16 * m * LDC + 16 * b, LDC, sdZ + 16 * m * LDB + 16 * jc, LDB, 16, lane);
        w -= sub;
        floatx4 u = zero4();
        Mma16<T>::mma(u, lds_col4<T>(sTd + b * 16 * LDD, LDD, 0, 0, lane), Mma16<T>::chain(w));
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * b + 4 * lg + r;
          sdZ[row * LDB + 16 * jc + lr] = from_float<T>(u[r]);
          sdZb[row * LDB + 16 * jc + lr] = from_float<T>(-vec[V_BETA * C + row] * vec[V_GAM * C + row] * u[r]);
          if (row < Lc) dzw[static_cast<size_t>(row) * v_tok] = u[r];
        }
      }
    }
    __syncthreads();
    // -- dM = gam_C dM' + s Q^T diag(gam) dO - K^T diag(beta gam) dZ
    {
      const float gC = vec[V_N * C];
#pragma unroll
      for (int i = 0; i < NMT; ++i) {
        const int t = wave + 4 * i, a = t / NJ, jc = t % NJ;
        dM[i] *= gC;
        tile_mm<T, true, true>(dM[i], sQ + 16 * a, LDK, sdOg + 16 * jc, LDB, C, lane);
        tile_mm<T, true, true>(dM[i], sK + 16 * a, LDK, sdZb + 16 * jc, LDB, C, lane);
      }
    }
    __syncthreads();
  }
  if (p.dh0) {
#pragma unroll
    for (int i = 0; i < NMT; ++i) {
      const int t = wave + 4 * i, a = t / NJ, jc = t % NJ;
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
  static constexpr int LDK = DK + PAD, LDV = DV + PAD, LDC = C + PAD;
  static constexpr int oQ = 0;
  static constexpr int oK = oQ + C * LDK * sizeof(T);
  static constexpr int odO = oK + C * LDK * sizeof(T);
  static constexpr int oU = odO + C * LDV * sizeof(T);
  static constexpr int odZ = oU + C * LDV * sizeof(T);
  static constexpr int oM = odZ + C * LDV * sizeof(T);  // M, then dM'
  static constexpr int odP = oM + DK * LDV * sizeof(T);
  static constexpr int oS = odP + C * LDC * sizeof(T);
  static constexpr int oVec = oS + C * LDC * sizeof(T);
  static constexpr int odG = oVec + (V_N * C + 4) * 4;
  static constexpr int odB = odG + C * 4;
  static constexpr int bytes = odB + C * 4;
};

template <class T, int DK, int DV>
__global__ __launch_bounds__(512) void dlocal_kernel(BwdParams p) {
  using L = DlLayout<T, DK, DV>;
  constexpr int LDK = L::LDK, LDV = L::LDV, LDC = L::LDC, NT = 512;
  constexpr int KTL = DK / 16;             // key-dim tiles
  constexpr int NOT = (C / 16) * KTL / 8;  // dq (and dk) tiles per wavefront
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
  float* sdG = reinterpret_cast<float*>(smem + L::odG);
  float* sdB = reinterpret_cast<float*>(smem + L::odB);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lg = lane >> 4, lr = lane & 15;
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
  const T* qg = static_cast<const T*>(p.q);
  const T* kg = static_cast<const T*>(p.k);
  const T* vg = static_cast<const T*>(p.v);
  const T* dog = static_cast<const T*>(p.dout);
  const float s = p.scale;

  stage_rows<T, T, DK>(sQ, LDK, qg + static_cast<size_t>(cs) * qk_tok + static_cast<size_t>(hq) * DK, qk_tok, Lc,
                       tid, NT);
  stage_rows<T, T, DK>(sK, LDK, kg + static_cast<size_t>(cs) * qk_tok + static_cast<size_t>(hq) * DK, qk_tok, Lc,
                       tid, NT);
  if (tid < C) {
    sdG[tid] = 0.f;
    sdB[tid] = 0.f;
  }
  __syncthreads();  // (the staging below adds into sdB)
  // output tiles of this wavefront: tile t = wave + 8i -> rows 16 (t / KTL), key columns 16 (t % KTL)
  floatx4 dqa[NOT], dka[NOT];
#pragma unroll
  for (int i = 0; i < NOT; ++i) dqa[i] = dka[i] = zero4();

  for (int hh = 0; hh < rep; ++hh) {
    const int h = hq * rep + hh;
    const size_t ck = (static_cast<size_t>(sq.cbase + c) * p.Hv + h) * DK * DV;
    // -- stage: dO, U, dZ, M; gates; dv = beta dZ and the dZ . v part of dbeta
    stage_rows<T, T, DV>(sdO, LDV, dog + static_cast<size_t>(cs) * v_tok + static_cast<size_t>(h) * DV, v_tok, Lc,
                         tid, NT);
    stage_rows<float, T, DV>(sU, LDV, p.ck_u + static_cast<size_t>(cs) * v_tok + static_cast<size_t>(h) * DV, v_tok,
                             Lc, tid, NT);
    for (int i = tid; i < DK * DV / 4; i += NT) {
      const int r = i / (DV / 4), e = (i - r * (DV / 4)) * 4;
      store4<T>(sM + r * LDV + e, load4(p.ck_state + ck + static_cast<size_t>(r) * DV + e));
    }
    if (wave == 0) {
      const size_t gi = static_cast<size_t>(cs) * p.Hv + h;
      gate_vectors(vec, p.g + gi, p.beta + gi, p.Hv, Lc, lane);
    }
    for (int i = tid; i < C * (DV / 4); i += NT) {  // 16 lanes per row when DV = 64, 32 when DV = 128
      const int t = i / (DV / 4), e = (i - t * (DV / 4)) * 4;
      floatx4 z = zero4(), vv = zero4();
      if (t < Lc) {
        const size_t off = static_cast<size_t>(cs + t) * v_tok + static_cast<size_t>(h) * DV + e;
        z = load4(p.dz + off);
        vv = load4(vg + off);
        const float bt = p.beta[static_cast<size_t>(cs + t) * p.Hv + h];
        *reinterpret_cast<floatx4*>(p.dv + off) = z * bt;
      }
      store4<T>(sdZ + t * LDV + e, z);
      float part = z[0] * vv[0] + z[1] * vv[1] + z[2] * vv[2] + z[3] * vv[3];
      if (t < Lc) atomicAdd(&sdB[t], part);
    }
    __syncthreads();
    // -- C x C tiles: dP (masked, times s exp(G_i - G_j)) and D + D^T; the M products
    for (int job = wave; job < 20; job += 8) {
      const int kind = job / 10, lt = job % 10;
      const int ti = lt < 1 ? 0 : lt < 3 ? 1 : lt < 6 ? 2 : 3;
      const int tj = lt - ti * (ti + 1) / 2;
      floatx4 gr = zero4(), d = zero4();
      tile_mm<T, false, false>(gr, (kind ? sK : sQ) + 16 * ti * LDK, LDK, sK + 16 * tj * LDK, LDK, DK, lane);
      tile_mm<T, false, false>(d, (kind ? sdZ : sdO) + 16 * ti * LDV, LDV, sU + 16 * tj * LDV, LDV, DV, lane);
      const int j = 16 * tj + lr;
      float colsum = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * ti + 4 * lg + r;
        const float dec = j <= i ? __builtin_amdgcn_exp2f(vec[V_GL * C + i] - vec[V_GL * C + j]) : 0.f;
        float w, rowb = 0.f;
        if (kind == 0) {  // P_ij = s dec (QK^T)_ij, dP_ij = (dO U^T)_ij, j <= i
          const bool on = j <= i;
          const float dp = on ? d[r] : 0.f;
          w = dp * s * dec * gr[r];
          sdP[i * LDC + j] = from_float<T>(dp * s * dec);
        } else {  // A_ij = beta_i dec (KK^T)_ij, dA_ij = -(dZ U^T)_ij, j < i
          const bool on = j < i;
          const float da = on ? -d[r] : 0.f;
          const float bi = vec[V_BETA * C + i];
          w = da * bi * dec * gr[r];
          rowb = da * dec * gr[r];
          const T dd = from_float<T>(da * bi * dec);
          if (on) {
            sS[i * LDC + j] = dd;
            sS[j * LDC + i] = dd;
          } else if (i == j) {
            sS[i * LDC + j] = from_float<T>(0.f);
          }
        }
        colsum += w;
        const float rw = sum16(w), rb = sum16(rowb);
        if (lr == 0) {
          atomicAdd(&sdG[i], rw);
          if (kind) atomicAdd(&sdB[i], rb);
        }
      }
      colsum += __shfl_xor(colsum, 16);
      colsum += __shfl_xor(colsum, 32);
      if (lg == 0) atomicAdd(&sdG[j], -colsum);
    }
#pragma unroll
    for (int i = 0; i < NOT; ++i) {
      const int t = wave + 8 * i, it = t / KTL, kt = t % KTL;
      floatx4 a = zero4(), b = zero4();
      tile_mm<T, false, false>(a, sdO + 16 * it * LDV, LDV, sM + 16 * kt * LDV, LDV, DV, lane);  // dO M^T
      tile_mm<T, false, false>(b, sdZ + 16 * it * LDV, LDV, sM + 16 * kt * LDV, LDV, DV, lane);  // dZ M^T
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * it + 4 * lg + r, key = 16 * kt + lr;
        const float gam = vec[V_GAM * C + row], bt = vec[V_BETA * C + row];
        dqa[i][r] += s * gam * a[r];
        dka[i][r] -= bt * gam * b[r];
        const float qa = sum16(to_float(sQ[row * LDK + key]) * a[r]);
        const float kb = sum16(to_float(sK[row * LDK + key]) * b[r]);
        if (lr == 0) {
          atomicAdd(&sdG[row], s * gam * qa - bt * gam * kb);
          atomicAdd(&sdB[row], -gam * kb);
        }
      }
    }
    __syncthreads();
    // -- dM' replaces M in LDS; gam_C <dM', M> enters dG at the chunk's end
    {
      float part = 0.f;
      const float* dmp = p.dm + ck;
      for (int i = tid; i < DK * DV / 4; i += NT) {
        const int r = i / (DV / 4), e = (i - r * (DV / 4)) * 4;
        const floatx4 dmv = load4(dmp + static_cast<size_t>(r) * DV + e);
        const floatx4 mv = load4(p.ck_state + ck + static_cast<size_t>(r) * DV + e);
        part += dmv[0] * mv[0] + dmv[1] * mv[1] + dmv[2] * mv[2] + dmv[3] * mv[3];
        store4<T>(sM + r * LDV + e, dmv);
      }
      part = sum16(part);
      part += __shfl_xor(part, 16);
      part += __shfl_xor(part, 32);
      if (lane == 0) atomicAdd(&sdG[C - 1], vec[V_N * C] * part);
    }
    __syncthreads();
    // -- dq += (dP s dec) K;  dk += diag(kf) U dM'^T + (dP s dec)^T Q + (D + D^T) K
#pragma unroll
    for (int i = 0; i < NOT; ++i) {
      const int t = wave + 8 * i, it = t / KTL, kt = t % KTL;
      tile_mm<T, false, true>(dqa[i], sdP + 16 * it * LDC, LDC, sK + 16 * kt, LDK, 16 * (it + 1), lane);
      floatx4 a = zero4();
      tile_mm<T, false, false>(a, sU + 16 * it * LDV, LDV, sM + 16 * kt * LDV, LDV, DV, lane);  // U dM'^T
      float ssum = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * it + 4 * lg + r, key = 16 * kt + lr;
        const float kf = vec[V_KF * C + row];
        dka[i][r] += kf * a[r];
        const float sj = kf * sum16(to_float(sK[row * LDK + key]) * a[r]);
        if (lr == 0) atomicAdd(&sdG[row], -sj);
        ssum += sj;
      }
      if (lr == 0) atomicAdd(&sdG[C - 1], ssum);
      tile_mm<T, true, true>(dka[i], sdP + 16 * it * LDC + 16 * it, LDC, sQ + 16 * it * LDK + 16 * kt, LDK,
                             C - 16 * it, lane);
      tile_mm<T, false, true>(dka[i], sS + 16 * it * LDC, LDC, sK + 16 * kt, LDK, C, lane);
    }
    __syncthreads();
    // -- dg = reverse cumsum of dG over the chunk; dbeta; clear the accumulators
    if (wave == 0) {
      const int t = C - 1 - lane;
      const float dg = wave_inclusive_sum(sdG[t]);
      const float db = sdB[t];
      if (t < Lc) {
        const size_t gi = static_cast<size_t>(cs + t) * p.Hv + h;
        p.dg[gi] = dg;
        p.dbeta[gi] = db;
      }
      sdG[t] = 0.f;
      sdB[t] = 0.f;
    }
    __syncthreads();
  }
  // dq, dk (summed over the value heads of this query/key head)
#pragma unroll
  for (int i = 0; i < NOT; ++i) {
    const int t = wave + 8 * i, it = t / KTL, kt = t % KTL;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 16 * it + 4 * lg + r;
      if (row < Lc) {
        const size_t off = static_cast<size_t>(cs + row) * qk_tok + static_cast<size_t>(hq) * DK + 16 * kt + lr;
        p.dq[off] = dqa[i][r];
        p.dk[off] = dka[i][r];
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

struct WsParts {
  size_t cpre, state, dm, u, dz, total;
};
WsParts ws_parts(int64_t tokens, int N, int Hv, int dk, int dv) {
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t chunks = static_cast<size_t>(tokens / C + N);
  WsParts w;
  w.cpre = 0;
  w.state = al(static_cast<size_t>(N + 1) * 4);
  w.dm = w.state + al(chunks * Hv * dk * dv * 4);
  w.u = w.dm + al(chunks * Hv * dk * dv * 4);
  w.dz = w.u + al(static_cast<size_t>(tokens) * Hv * dv * 4);
  w.total = w.dz + al(static_cast<size_t>(tokens) * Hv * dv * 4);
  return w;
}

template <class T, int DK, int DV, int BV>
hipError_t launch(const BwdArgs& a, hipStream_t stream) {
  using LS = DsLayout<T, DK, BV>;
  using LL = DlLayout<T, DK, DV>;
  static_assert(LS::bytes <= 160 * 1024 && LL::bytes <= 160 * 1024, "LDS budget of one gfx950 compute unit");
  const int64_t tokens = static_cast<int64_t>(a.batch) * a.seqlen;
  const WsParts w = ws_parts(tokens, a.num_seqs, a.Hv, DK, DV);
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
  f.save_state = reinterpret_cast<float*>(ws + w.state);
  f.save_u = reinterpret_cast<float*>(ws + w.u);
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
  p.dm = reinterpret_cast<float*>(ws + w.dm);
  p.dz = reinterpret_cast<float*>(ws + w.dz);
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
  dstate_kernel<T, DK, DV, BV><<<dim3(units * (DV / BV)), dim3(256), LS::bytes, stream>>>(p);
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(&dlocal_kernel<T, DK, DV>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, LL::bytes);
  if (e != hipSuccess) return e;
  dlocal_kernel<T, DK, DV><<<dim3(p.chunk_bound * a.Hqk), dim3(512), LL::bytes, stream>>>(p);
  return hipGetLastError();
}

}  // namespace

size_t bwd_workspace_bytes(int64_t tokens, int num_seqs, int Hv, int dk, int dv) {
  return ws_parts(tokens, num_seqs, Hv, dk, dv).total;
}

hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream) {
  if (a.bf16) {
    if (a.head_dim_k == 128 && a.head_dim_v == 128) return launch<bf16, 128, 128, 32>(a, stream);
    if (a.head_dim_k == 64 && a.head_dim_v == 64) return launch<bf16, 64, 64, 32>(a, stream);
  } else {
    if (a.head_dim_k == 64 && a.head_dim_v == 64) return launch<float, 64, 64, 32>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdn

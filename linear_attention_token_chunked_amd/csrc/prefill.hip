// Chunked-parallel prefill of the gated delta rule on gfx950.
//
// Method: the recurrence from the podcast transcript on "On the Design of
// Qwen3.8-Next Architecture", cue 14 (decay the whole state, read what the key
// holds, write only the error), in the stored layout M = S^T (dk x dv).  Inside
// a chunk of C = 64 tokens that starts from state M, unrolling the recurrence
// gives the UT/WY form (G = inclusive in-chunk cumsum of g = log alpha):
//   A   = strict_lower(beta_i exp(G_i - G_j) (K K^T)_ij)        (C x C)
//   T   = (I + A)^-1                                             (unit lower)
//   W   = T diag(beta exp G) K,   Ut = T diag(beta) V
//   U   = Ut - W M                                               (C x dv)
//   O   = scale (diag(exp G) Q M + lower_incl(exp(G_i - G_j) (Q K^T)_ij) U)
//   M  <- exp(G_C) M + K^T diag(exp(G_C - G)) U
// which is exact in real arithmetic.
//
// Kernel structure.  One workgroup (4 wavefronts) owns one (sequence, value
// head, dv-slice) and walks its chunks in order, holding the fp32 state slice
// in registers the whole time, so the state never touches HBM between chunks
// and no workspace exists.  Per chunk:
//   phase 0  gates (wave-level prefix sum), K, K^T, Q, V^T of the chunk -> LDS
//   phase 1  K K^T and Q K^T on the matrix cores, masked with the decay -> A, P
//   phase 2  16x16 diagonal blocks of (I + A)^-1 by forward substitution (fp32)
//   phase 3  off-diagonal blocks, block row by block row (fp32 matrix cores)
//   phase 4  T diag(beta exp G), T diag(beta) as matrix-core operands
//   phase 5  W (negated) = T diag(beta exp G) K
//   phase 6  per wavefront, on its own dv columns: Ut, U = Ut - W M, the output
//            tile O^T, and the state update; here the state and U are fed to
//            the next product straight from the accumulator registers.
// bf16 inputs use v_mfma_f32_16x16x32_bf16 with fp32 accumulation (the state
// is rounded to bf16 only as an operand); fp32 inputs use v_mfma_f32_16x16x4_f32
// so that nothing is rounded below fp32.  The triangular solve is fp32 in both.
#include "device_common.hpp"
#include "launch.hpp"

namespace gdn {
namespace {

constexpr int C = 64;            // chunk length
constexpr int NW = 4;            // wavefronts per workgroup
constexpr int NTHREADS = 64 * NW;

template <class T, int DK, int BV>
struct Layout {
  static constexpr int EPB = 16 / sizeof(T);   // elements per 16 bytes
  static constexpr int NTW = BV / (16 * NW);   // 16-column tiles per wavefront
  static constexpr int LDK = DK + EPB;         // row stride of [C][DK] tiles: sK, sQ, sW
  static constexpr int LDC = C + EPB;          // row stride of [*][C] tiles: sKT, sVT, sTw, sTu, sP
  static constexpr int LDF = C + 4;            // row stride of the fp32 [C][C] tiles: sA, sT
  static constexpr size_t oK = 0;
  static constexpr size_t oQ = oK + sizeof(T) * C * LDK;
  static constexpr size_t oKT = oQ + sizeof(T) * C * LDK;
  static constexpr size_t oVT = oKT + sizeof(T) * DK * LDC;
  static constexpr size_t oTw = oVT + sizeof(T) * BV * LDC;
  static constexpr size_t oTu = oTw + sizeof(T) * C * LDC;
  static constexpr size_t oP = oTu + sizeof(T) * C * LDC;
  static constexpr size_t oA = oP + sizeof(T) * C * LDC;  // fp32 A; reused for W after the solve
  static constexpr size_t szA = (4 * C * LDF > sizeof(T) * C * LDK) ? 4 * C * LDF : sizeof(T) * C * LDK;
  static constexpr size_t oT = oA + szA;
  static constexpr size_t oV = oT + 4 * C * LDF;         // five per-token fp32 vectors
  static constexpr size_t bytes = oV + 4 * 5 * C;
  static_assert(BV % (16 * NW) == 0, "dv-slice must give every wavefront whole 16-column tiles");
  static_assert(oQ % 16 == 0 && oKT % 16 == 0 && oVT % 16 == 0 && oTw % 16 == 0 && oP % 16 == 0 &&
                oA % 16 == 0 && oT % 16 == 0 && oV % 16 == 0, "16-byte aligned LDS regions");
};

struct Params {
  const void *q, *k, *v;
  const float *g, *beta, *h0;
  const int32_t* cu;
  void* o;
  float* hT;
  int T, Hqk, Hv, nunits, nslices;
  float scale;
};

// Logical contraction index stored at LDS position P (inverse of phys_k).
template <class T>
__device__ __forceinline__ int logical_k(int P);
template <>
__device__ __forceinline__ int logical_k<bf16>(int P) {
  return (P & ~31) | (((P >> 2) & 1) << 4) | (((P >> 3) & 3) << 2) | (P & 3);
}
template <>
__device__ __forceinline__ int logical_k<float>(int P) { return P; }

// Operand fragment of k-group kg built from accumulator tiles tile(kg*TPG + t).
template <class T, class F>
__device__ __forceinline__ typename Mma<T>::frag chain_frag(F tile, int kg) {
  if constexpr (Mma<T>::TPG == 2) {
    return Mma<T>::chain(tile(2 * kg), tile(2 * kg + 1));
  } else {
    return Mma<float>::chain(tile(kg));
  }
}

template <class T>
struct Raw16 {  // 16 bytes of T
  typename Mma<T>::frag v;
};

template <class T, int DK, int DV, int BV>
__global__ __launch_bounds__(NTHREADS, 1) void prefill_kernel(Params p) {
  using L = Layout<T, DK, BV>;
  using MM = Mma<T>;
  using frag = typename MM::frag;
  using V4 = typename Vec4<T>::type;
  constexpr int EPB = L::EPB, NTW = L::NTW, LDK = L::LDK, LDC = L::LDC, LDF = L::LDF;
  constexpr int KT = DK / 16;  // key-dim tiles of the state

  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  T* sK = reinterpret_cast<T*>(smem + L::oK);
  T* sQ = reinterpret_cast<T*>(smem + L::oQ);
  T* sKT = reinterpret_cast<T*>(smem + L::oKT);
  T* sVT = reinterpret_cast<T*>(smem + L::oVT);
  T* sTw = reinterpret_cast<T*>(smem + L::oTw);
  T* sTu = reinterpret_cast<T*>(smem + L::oTu);
  T* sP = reinterpret_cast<T*>(smem + L::oP);
  float* sA = reinterpret_cast<float*>(smem + L::oA);
  T* sW = reinterpret_cast<T*>(smem + L::oA);
  float* sT = reinterpret_cast<float*>(smem + L::oT);
  float* sG = reinterpret_cast<float*>(smem + L::oV);  // G
  float* seG = sG + C;                                 // exp(G)
  float* segl = seG + C;                               // exp(G_C - G)
  float* sb = segl + C;                                // beta
  float* sbg = sb + C;                                 // beta exp(G)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lg = lane >> 4;  // lane group: accumulator rows 4lg..4lg+3
  const int lr = lane & 15;  // lane row / column inside a 16x16 tile

  // Workgroup -> (unit, dv-slice).  Consecutive workgroups are dealt to the 8
  // XCDs in turn, so the slices of one unit (which read the same q/k/v chunks)
  // are given ids 8 apart and land on the same XCD and its L2.
  const int xcd = blockIdx.x & 7;
  const int rest = blockIdx.x >> 3;
  const int slice = rest % p.nslices;
  const int unit = xcd + 8 * (rest / p.nslices);
  if (unit >= p.nunits) return;
  const int n = unit / p.Hv;
  const int h = unit - n * p.Hv;
  const int hq = h / (p.Hv / p.Hqk);
  int bos, eos;
  if (p.cu) {
    bos = p.cu[n];
    eos = p.cu[n + 1];
  } else {
    bos = n * p.T;
    eos = bos + p.T;
  }
  const int col0 = slice * BV;                 // first value column of the workgroup
  const int wcol = col0 + wave * 16 * NTW;     // first value column of this wavefront

  const T* qg = static_cast<const T*>(p.q);
  const T* kg_ = static_cast<const T*>(p.k);
  const T* vg = static_cast<const T*>(p.v);
  T* og = static_cast<T*>(p.o);
  const size_t qk_tok = static_cast<size_t>(p.Hqk) * DK;  // token stride of q, k
  const size_t v_tok = static_cast<size_t>(p.Hv) * DV;    // token stride of v, o

  // State tiles: Ms[a][j] holds M[16a + 4lg + s][wcol + 16j + lr], s = 0..3.
  floatx4 Ms[KT][NTW];
  const size_t sbase = static_cast<size_t>(unit) * DK * DV;
#pragma unroll
  for (int a = 0; a < KT; ++a)
#pragma unroll
    for (int j = 0; j < NTW; ++j)
#pragma unroll
      for (int s = 0; s < 4; ++s)
        Ms[a][j][s] = p.h0 ? p.h0[sbase + static_cast<size_t>(16 * a + 4 * lg + s) * DV + wcol + 16 * j + lr]
                           : 0.f;

  for (int cs = bos; cs < eos; cs += C) {
    const int Lc = min(C, eos - cs);

    // ---------------- phase 0: gates and operand tiles into LDS ----------------
    if (wave == 0) {
      float gt = 0.f, bt = 0.f;  // tokens past the end act as g = 0, beta = 0 (no-ops)
      if (lane < Lc) {
        gt = p.g[static_cast<size_t>(cs + lane) * p.Hv + h];
        bt = p.beta[static_cast<size_t>(cs + lane) * p.Hv + h];
      }
      float G = gt;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(G, off);
        if (lane >= off) G += y;
      }
      const float GC = __shfl(G, 63);
      const float eG = expf(G);
      sG[lane] = G;
      seG[lane] = eG;
      segl[lane] = expf(GC - G);
      sb[lane] = bt;
      sbg[lane] = bt * eG;
    }
    {
      // K: row layout (sK) and transposed (sKT) from one pass of loads.  A task
      // reads the EPB token rows that sit at LDS positions [EPB*pg, EPB*pg+EPB)
      // of sKT's token axis and EPB key columns, then writes both layouts.
      constexpr int NPG = C / EPB, NCG = DK / EPB;
      const T* kb = kg_ + static_cast<size_t>(cs) * qk_tok + static_cast<size_t>(hq) * DK;
      for (int task = tid; task < NPG * NCG; task += NTHREADS) {
        const int pg = task / NCG, cgp = task - (task / NCG) * NCG;
        Raw16<T> rows[EPB];
#pragma unroll
        for (int e = 0; e < EPB; ++e) {
          const int r = logical_k<T>(pg * EPB + e);
          if (r < Lc) {
            rows[e].v = *reinterpret_cast<const frag*>(kb + r * qk_tok + cgp * EPB);
          } else {
#pragma unroll
            for (int c = 0; c < EPB; ++c) rows[e].v[c] = from_float<T>(0.f);
          }
#pragma unroll
          for (int u = 0; u < EPB / 4; ++u) {
            V4 w4;
#pragma unroll
            for (int c = 0; c < 4; ++c) w4[c] = rows[e].v[4 * u + c];
            *reinterpret_cast<V4*>(sK + r * LDK + MM::phys_k(cgp * EPB + 4 * u)) = w4;
          }
        }
#pragma unroll
        for (int c = 0; c < EPB; ++c) {
          Raw16<T> col;
#pragma unroll
          for (int e = 0; e < EPB; ++e) col.v[e] = rows[e].v[c];
          *reinterpret_cast<frag*>(sKT + (cgp * EPB + c) * LDC + pg * EPB) = col.v;
        }
      }
      // Q: row layout only.
      const T* qb = qg + static_cast<size_t>(cs) * qk_tok + static_cast<size_t>(hq) * DK;
      for (int task = tid; task < C * NCG; task += NTHREADS) {
        const int r = task / NCG, cgp = task - (task / NCG) * NCG;
        Raw16<T> x;
        if (r < Lc) {
          x.v = *reinterpret_cast<const frag*>(qb + r * qk_tok + cgp * EPB);
        } else {
#pragma unroll
          for (int c = 0; c < EPB; ++c) x.v[c] = from_float<T>(0.f);
        }
#pragma unroll
        for (int u = 0; u < EPB / 4; ++u) {
          V4 w4;
#pragma unroll
          for (int c = 0; c < 4; ++c) w4[c] = x.v[4 * u + c];
          *reinterpret_cast<V4*>(sQ + r * LDK + MM::phys_k(cgp * EPB + 4 * u)) = w4;
        }
      }
      // V: this workgroup's dv-slice, transposed.
      constexpr int NVG = BV / EPB;
      const T* vb = vg + static_cast<size_t>(cs) * v_tok + static_cast<size_t>(h) * DV + col0;
      for (int task = tid; task < NPG * NVG; task += NTHREADS) {
        const int pg = task / NVG, cgp = task - (task / NVG) * NVG;
        Raw16<T> rows[EPB];
#pragma unroll
        for (int e = 0; e < EPB; ++e) {
          const int r = logical_k<T>(pg * EPB + e);
          if (r < Lc) {
            rows[e].v = *reinterpret_cast<const frag*>(vb + r * v_tok + cgp * EPB);
          } else {
#pragma unroll
            for (int c = 0; c < EPB; ++c) rows[e].v[c] = from_float<T>(0.f);
          }
        }
#pragma unroll
        for (int c = 0; c < EPB; ++c) {
          Raw16<T> col;
#pragma unroll
          for (int e = 0; e < EPB; ++e) col.v[e] = rows[e].v[c];
          *reinterpret_cast<frag*>(sVT + (cgp * EPB + c) * LDC + pg * EPB) = col.v;
        }
      }
    }
    __syncthreads();

    // ---------------- phase 1: K K^T and Q K^T, masked with the decay ----------------
    {
      // Wavefront w owns token rows i in [16w, 16w+16).  Tile c of both products
      // is computed transposed so that a lane ends up holding four consecutive
      // columns j = 16c + 4lg + s of row i = 16w + lr.
      const int w = wave;
      floatx4 kk[4], qk[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) kk[c] = qk[c] = zero4();
#pragma unroll
      for (int kgi = 0; kgi < DK / MM::KG; ++kgi) {
        const frag bk = lds_frag(sK + (16 * w + lr) * LDK, kgi, lane);
        const frag bq = lds_frag(sQ + (16 * w + lr) * LDK, kgi, lane);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          if (c <= w) {  // only tiles on or below the diagonal are needed
            const frag a = lds_frag(sK + (16 * c + lr) * LDK, kgi, lane);
            MM::mma(kk[c], a, bk);
            MM::mma(qk[c], a, bq);
          }
        }
      }
      const int i = 16 * w + lr;
      const float Gi = sG[i], bi = sb[i];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        floatx4 av = zero4(), pv = zero4();
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int j = 16 * c + 4 * lg + s;
          if (j <= i) {  // exp(G_i - G_j) is formed only on and below the diagonal
            const float d = expf(Gi - sG[j]);
            av[s] = (j < i) ? bi * d * kk[c][s] : 0.f;
            pv[s] = d * qk[c][s];
          }
        }
        *reinterpret_cast<floatx4*>(sA + i * LDF + 16 * c + 4 * lg) = av;
        *reinterpret_cast<V4*>(sP + i * LDC + MM::phys_k(16 * c + 4 * lg)) = pack4<T>(pv[0], pv[1], pv[2], pv[3]);
      }
    }
    __syncthreads();

    // ---------------- phase 2: diagonal 16x16 blocks of (I + A)^-1 ----------------
    if (wave == 0) {
      // Lane (blk, cc) computes column cc of the inverse of block blk by forward
      // substitution: x_i = [i == cc] - sum_{j < i} A_ij x_j.
      const int blk = lg, cc = lr;
      const float* Ab = sA + (16 * blk) * LDF + 16 * blk;
      float x[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float acc = (i == cc) ? 1.f : 0.f;
#pragma unroll
        for (int j = 0; j < i; ++j) acc -= Ab[i * LDF + j] * x[j];
        x[i] = acc;
      }
      float* Tb = sT + (16 * blk) * LDF + 16 * blk;
#pragma unroll
      for (int i = 0; i < 16; ++i) Tb[i * LDF + cc] = x[i];
    }
    __syncthreads();

    // ---------------- phase 3: off-diagonal blocks, one block diagonal at a time ----------------
    // T_ij = -T_ii * sum_{m=j}^{i-1} A_im T_mj   (16x16 blocks, i > j)
#pragma unroll
    for (int d = 1; d < 4; ++d) {
      if (wave < 4 - d) {
        const int bj = wave, bi = wave + d;
        floatx4 y = zero4();
        for (int m = bj; m < bi; ++m) {
          const floatx4 af = *reinterpret_cast<const floatx4*>(sA + (16 * bi + lr) * LDF + 16 * m + 4 * lg);
          floatx4 bf;
#pragma unroll
          for (int s = 0; s < 4; ++s) bf[s] = sT[(16 * m + 4 * lg + s) * LDF + 16 * bj + lr];
          Mma<float>::mma(y, af, bf);
        }
        const floatx4 tf = *reinterpret_cast<const floatx4*>(sT + (16 * bi + lr) * LDF + 16 * bi + 4 * lg);
        floatx4 t = zero4();
        Mma<float>::mma(t, tf, y);
#pragma unroll
        for (int s = 0; s < 4; ++s) sT[(16 * bi + 4 * lg + s) * LDF + 16 * bj + lr] = -t[s];
      }
      __syncthreads();
    }

    // ---------------- phase 4: T diag(beta exp G) and T diag(beta) as operands ----------------
    for (int task = tid; task < C * (C / 4); task += NTHREADS) {
      const int i = task / (C / 4), j0 = 4 * (task - (task / (C / 4)) * (C / 4));
      floatx4 t = zero4();
      if ((j0 >> 4) <= (i >> 4)) t = *reinterpret_cast<const floatx4*>(sT + i * LDF + j0);
      *reinterpret_cast<V4*>(sTw + i * LDC + MM::phys_k(j0)) =
          pack4<T>(t[0] * sbg[j0], t[1] * sbg[j0 + 1], t[2] * sbg[j0 + 2], t[3] * sbg[j0 + 3]);
      *reinterpret_cast<V4*>(sTu + i * LDC + MM::phys_k(j0)) =
          pack4<T>(t[0] * sb[j0], t[1] * sb[j0 + 1], t[2] * sb[j0 + 2], t[3] * sb[j0 + 3]);
    }
    __syncthreads();

    // ---------------- phase 5: -W = -(T diag(beta exp G)) K, computed as W^T ----------------
    {
      const int w = wave;  // W rows 16w..16w+15
      floatx4 acc[KT];
#pragma unroll
      for (int a = 0; a < KT; ++a) acc[a] = zero4();
#pragma unroll
      for (int kgi = 0; kgi < C / MM::KG; ++kgi) {
        const frag bt = lds_frag(sTw + (16 * w + lr) * LDC, kgi, lane);
#pragma unroll
        for (int a = 0; a < KT; ++a) MM::mma(acc[a], lds_frag(sKT + (16 * a + lr) * LDC, kgi, lane), bt);
      }
      // lane holds W[16w + lr][16a + 4lg + s]
#pragma unroll
      for (int a = 0; a < KT; ++a)
        *reinterpret_cast<V4*>(sW + (16 * w + lr) * LDK + MM::phys_k(16 * a + 4 * lg)) =
            pack4<T>(-acc[a][0], -acc[a][1], -acc[a][2], -acc[a][3]);
    }
    __syncthreads();

    // ---------------- phase 6: per-wavefront state work on its own dv columns ----------------
    {
      // U tiles: U[r][j] holds U[16r + 4lg + s][wcol + 16j + lr].
      floatx4 U[4][NTW];
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int j = 0; j < NTW; ++j) U[r][j] = zero4();
      // Ut = T diag(beta) V
#pragma unroll
      for (int kgi = 0; kgi < C / MM::KG; ++kgi) {
        frag bv[NTW];
#pragma unroll
        for (int j = 0; j < NTW; ++j) bv[j] = lds_frag(sVT + ((wave * NTW + j) * 16 + lr) * LDC, kgi, lane);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const frag af = lds_frag(sTu + (16 * r + lr) * LDC, kgi, lane);
#pragma unroll
          for (int j = 0; j < NTW; ++j) MM::mma(U[r][j], af, bv[j]);
        }
      }
      // U = Ut + (-W) M, with M fed from the state registers
#pragma unroll
      for (int kgi = 0; kgi < DK / MM::KG; ++kgi) {
        frag bm[NTW];
#pragma unroll
        for (int j = 0; j < NTW; ++j) bm[j] = chain_frag<T>([&](int t) { return Ms[t][j]; }, kgi);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const frag af = lds_frag(sW + (16 * r + lr) * LDK, kgi, lane);
#pragma unroll
          for (int j = 0; j < NTW; ++j) MM::mma(U[r][j], af, bm[j]);
        }
      }
      // O^T = M^T Q^T diag(exp G) + U^T P^T, one 16x16 tile per (own n-tile j, token tile c)
#pragma unroll
      for (int j = 0; j < NTW; ++j) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          floatx4 acc = zero4();
#pragma unroll
          for (int kgi = 0; kgi < DK / MM::KG; ++kgi)
            MM::mma(acc, chain_frag<T>([&](int t) { return Ms[t][j]; }, kgi),
                    lds_frag(sQ + (16 * c + lr) * LDK, kgi, lane));
          acc *= seG[16 * c + lr];
#pragma unroll
          for (int kgi = 0; kgi < C / MM::KG; ++kgi)
            MM::mma(acc, chain_frag<T>([&](int t) { return U[t][j]; }, kgi),
                    lds_frag(sP + (16 * c + lr) * LDC, kgi, lane));
          acc *= p.scale;
          // lane holds O[token 16c + lr][wcol + 16j + 4lg + s]
          const int tok = 16 * c + lr;
          if (tok < Lc)
            *reinterpret_cast<V4*>(og + static_cast<size_t>(cs + tok) * v_tok + static_cast<size_t>(h) * DV + wcol +
                                   16 * j + 4 * lg) = pack4<T>(acc[0], acc[1], acc[2], acc[3]);
        }
      }
      // M <- exp(G_C) M + K^T (diag(exp(G_C - G)) U)
      const float eGC = seG[C - 1];
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const float f = segl[16 * r + 4 * lg + s];
#pragma unroll
          for (int j = 0; j < NTW; ++j) U[r][j][s] *= f;
        }
#pragma unroll
      for (int a = 0; a < KT; ++a)
#pragma unroll
        for (int j = 0; j < NTW; ++j) Ms[a][j] *= eGC;
#pragma unroll
      for (int kgi = 0; kgi < C / MM::KG; ++kgi) {
        frag bu[NTW];
#pragma unroll
        for (int j = 0; j < NTW; ++j) bu[j] = chain_frag<T>([&](int t) { return U[t][j]; }, kgi);
#pragma unroll
        for (int a = 0; a < KT; ++a) {
          const frag af = lds_frag(sKT + (16 * a + lr) * LDC, kgi, lane);
#pragma unroll
          for (int j = 0; j < NTW; ++j) MM::mma(Ms[a][j], af, bu[j]);
        }
      }
    }
    __syncthreads();  // the next chunk overwrites every LDS tile
  }

  if (p.hT) {
#pragma unroll
    for (int a = 0; a < KT; ++a)
#pragma unroll
      for (int j = 0; j < NTW; ++j)
#pragma unroll
        for (int s = 0; s < 4; ++s)
          p.hT[sbase + static_cast<size_t>(16 * a + 4 * lg + s) * DV + wcol + 16 * j + lr] = Ms[a][j][s];
  }
}

template <class T, int DK, int DV, int BV>
hipError_t launch(const PrefillArgs& a, hipStream_t stream) {
  using L = Layout<T, DK, BV>;
  Params p;
  p.q = a.q;
  p.k = a.k;
  p.v = a.v;
  p.g = a.g;
  p.beta = a.beta;
  p.h0 = a.initial_state;
  p.cu = a.cu_seqlens;
  p.o = a.o;
  p.hT = a.final_state;
  p.T = a.seqlen;
  p.Hqk = a.Hqk;
  p.Hv = a.Hv;
  p.nunits = a.num_seqs * a.Hv;
  p.nslices = DV / BV;
  p.scale = a.scale;
  if (p.nunits == 0) return hipSuccess;
  const int units_pad = (p.nunits + 7) / 8 * 8;
  const dim3 grid(units_pad * p.nslices);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_kernel<T, DK, DV, BV>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(L::bytes));
  if (e != hipSuccess) return e;
  prefill_kernel<T, DK, DV, BV><<<grid, dim3(NTHREADS), L::bytes, stream>>>(p);
  return hipGetLastError();
}

// dv-slice width: whole state rows per workgroup when there are enough
// (sequence, head) units to fill the 256 compute units, narrower slices
// (more workgroups, each redoing the chunk-local work) when there are not.
int choose_bv(int units, int dv) {
  if (dv == 64) return 64;
  return units >= 256 ? 128 : 64;
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  if (a.chunk != C) return hipErrorInvalidValue;
  const int units = a.num_seqs * a.Hv;
  if (a.bf16) {
    if (a.dk == 128 && a.dv == 128)
      return choose_bv(units, 128) == 128 ? launch<bf16, 128, 128, 128>(a, stream)
                                          : launch<bf16, 128, 128, 64>(a, stream);
    if (a.dk == 64 && a.dv == 64) return launch<bf16, 64, 64, 64>(a, stream);
  } else {
    if (a.dk == 64 && a.dv == 64) return launch<float, 64, 64, 64>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdn

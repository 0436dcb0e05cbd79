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
//   phase 0  the chunk's K, K^T, Q, V^T and gate prefix sums -> LDS (the global
//            loads were issued one chunk earlier and are already in registers);
//            the next chunk's loads are issued here and land during phases 1-6
//   phase 1  K K^T and Q K^T on the matrix cores, masked with the decay -> A, P
//   phase 2  16x16 diagonal blocks of (I + A)^-1 by forward substitution (fp32)
//   phase 3  off-diagonal blocks, one block diagonal at a time (fp32 matrix
//            cores); a transposed copy of T lives above the diagonal of A
//   phase 4  T diag(beta exp G), T diag(beta) as matrix-core operands
//   phase 5  W (negated) = T diag(beta exp G) K
//   phase 6  per wavefront, on its own dv columns: Ut, U = Ut - W M, the output
//            tile O^T, and the state update; here the state and U are fed to
//            the next product straight from the accumulator registers.
// bf16 inputs use v_mfma_f32_16x16x32_bf16 with fp32 accumulation (the state
// is rounded to bf16 only as an operand); fp32 inputs use v_mfma_f32_16x16x4_f32
// so that nothing is rounded below fp32.  The triangular solve is fp32 in both.
// Decay factors are exp2 of log2(e)-scaled prefix sums, and exp(G_i - G_j) is
// only ever formed for i >= j, where it is at most 1 for decaying gates.
#include "device_common.hpp"
#include "launch.hpp"

namespace gdn {
namespace {

constexpr int C = 64;            // chunk length
constexpr int NW = 4;            // wavefronts per workgroup
constexpr int NTHREADS = 64 * NW;
constexpr float kLog2e = 1.4426950408889634f;

template <class T, int DK, int BV>
struct Layout {
  static constexpr int EPB = 16 / sizeof(T);   // elements per 16 bytes
  static constexpr int NTW = BV / (16 * NW);   // 16-column tiles per wavefront
  static constexpr int LDK = DK + EPB;         // row stride of [C][DK] tiles: sK / sW, sQ
  static constexpr int LDC = C + EPB;          // row stride of [*][C] tiles: sKT, sVT, sTw, sTu, sP
  static constexpr int LDF = C + 4;            // row stride of the fp32 [C][C] tiles: sA, sT
  static constexpr size_t oK = 0;              // K rows; reused for -W once the Gram products are done
  static constexpr size_t oQ = oK + sizeof(T) * C * LDK;
  static constexpr size_t oKT = oQ + sizeof(T) * C * LDK;
  static constexpr size_t oVT = oKT + sizeof(T) * DK * LDC;
  static constexpr size_t oTw = oVT + sizeof(T) * BV * LDC;
  static constexpr size_t oTu = oTw + sizeof(T) * C * LDC;
  static constexpr size_t oP = oTu + sizeof(T) * C * LDC;
  static constexpr size_t oA = oP + sizeof(T) * C * LDC;  // fp32: A below the diagonal, T^T on and above
  static constexpr size_t oT = oA + 4 * C * LDF;          // fp32: T row-major
  static constexpr size_t oV = oT + 4 * C * LDF;          // five per-token fp32 vectors
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
__device__ __forceinline__ typename Mma<T>::frag zero_frag() {
  typename Mma<T>::frag z;
#pragma unroll
  for (int i = 0; i < 16 / static_cast<int>(sizeof(T)); ++i) z[i] = from_float<T>(0.f);
  return z;
}

// The raw operands of one chunk, held in registers between the global loads
// (issued one chunk ahead) and the LDS stores.  Tokens past the end of the
// sequence load as zeros, and their gates as g = 0, beta = 0, which makes
// them exact no-ops in every product.
template <class T, int DK, int BV>
struct ChunkRegs {
  typedef typename Mma<T>::frag frag;
  static constexpr int EPB = 16 / sizeof(T);
  static constexpr int NKT = (C / 4) * (DK / EPB);  // K tasks: 4 token rows x EPB key columns
  static constexpr int KIT = (NKT + NTHREADS - 1) / NTHREADS;
  static constexpr int NQP = C * (DK / EPB);        // Q 16-byte pieces
  static constexpr int QIT = (NQP + NTHREADS - 1) / NTHREADS;
  static constexpr int NVT = (C / 4) * (BV / EPB);  // V tasks: 4 token rows x EPB value columns
  static constexpr int VIT = (NVT + NTHREADS - 1) / NTHREADS;
  frag k[KIT][4];
  frag q[QIT];
  frag v[VIT][4];
  float g, b;

  // kb, qb, vb point at the chunk's first token (head and column offsets applied).
  __device__ __forceinline__ void load(const T* kb, const T* qb, const T* vb, size_t qk_tok, size_t v_tok,
                                       const float* gb, const float* bb, size_t g_tok, int Lc, int tid) {
#pragma unroll
    for (int it = 0; it < KIT; ++it) {
      const int t = tid + it * NTHREADS;
      const int rg = t % (C / 4), cgp = t / (C / 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * rg + e;
        k[it][e] = (t < NKT && r < Lc) ? *reinterpret_cast<const frag*>(kb + r * qk_tok + cgp * EPB)
                                       : zero_frag<T>();
      }
    }
#pragma unroll
    for (int it = 0; it < QIT; ++it) {
      const int t = tid + it * NTHREADS;
      const int r = t / (DK / EPB), cgp = t % (DK / EPB);
      q[it] = (t < NQP && r < Lc) ? *reinterpret_cast<const frag*>(qb + r * qk_tok + cgp * EPB) : zero_frag<T>();
    }
#pragma unroll
    for (int it = 0; it < VIT; ++it) {
      const int t = tid + it * NTHREADS;
      const int rg = t % (C / 4), cgp = t / (C / 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * rg + e;
        v[it][e] = (t < NVT && r < Lc) ? *reinterpret_cast<const frag*>(vb + r * v_tok + cgp * EPB)
                                       : zero_frag<T>();
      }
    }
    g = 0.f;
    b = 0.f;
    if (tid < 64 && tid < Lc) {
      g = gb[tid * g_tok];
      b = bb[tid * g_tok];
    }
  }

  // K -> sK (row layout) and sKT (transposed), Q -> sQ, V -> sVT (transposed).
  // Contraction axes are stored in phys_k order (see device_common.hpp).
  __device__ __forceinline__ void store(T* sK, T* sKT, T* sQ, T* sVT, int LDK, int LDC, int tid) const {
    typedef typename Vec4<T>::type V4;
#pragma unroll
    for (int it = 0; it < KIT; ++it) {
      const int t = tid + it * NTHREADS;
      if (t < NKT) {
        const int rg = t % (C / 4), cgp = t / (C / 4);
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int u = 0; u < EPB / 4; ++u) {
            V4 w4;
#pragma unroll
            for (int c = 0; c < 4; ++c) w4[c] = k[it][e][4 * u + c];
            *reinterpret_cast<V4*>(sK + (4 * rg + e) * LDK + Mma<T>::phys_k(cgp * EPB + 4 * u)) = w4;
          }
#pragma unroll
        for (int c = 0; c < EPB; ++c) {
          V4 col;
#pragma unroll
          for (int e = 0; e < 4; ++e) col[e] = k[it][e][c];
          *reinterpret_cast<V4*>(sKT + (cgp * EPB + c) * LDC + Mma<T>::phys_k(4 * rg)) = col;
        }
      }
    }
#pragma unroll
    for (int it = 0; it < QIT; ++it) {
      const int t = tid + it * NTHREADS;
      if (t < NQP) {
        const int r = t / (DK / EPB), cgp = t % (DK / EPB);
#pragma unroll
        for (int u = 0; u < EPB / 4; ++u) {
          V4 w4;
#pragma unroll
          for (int c = 0; c < 4; ++c) w4[c] = q[it][4 * u + c];
          *reinterpret_cast<V4*>(sQ + r * LDK + Mma<T>::phys_k(cgp * EPB + 4 * u)) = w4;
        }
      }
    }
#pragma unroll
    for (int it = 0; it < VIT; ++it) {
      const int t = tid + it * NTHREADS;
      if (t < NVT) {
        const int rg = t % (C / 4), cgp = t / (C / 4);
#pragma unroll
        for (int c = 0; c < EPB; ++c) {
          V4 col;
#pragma unroll
          for (int e = 0; e < 4; ++e) col[e] = v[it][e][c];
          *reinterpret_cast<V4*>(sVT + (cgp * EPB + c) * LDC + Mma<T>::phys_k(4 * rg)) = col;
        }
      }
    }
  }
};

template <class T, int DK, int DV, int BV>
__global__ __launch_bounds__(NTHREADS, 1) void prefill_kernel(Params p) {
  using L = Layout<T, DK, BV>;
  using MM = Mma<T>;
  using frag = typename MM::frag;
  using V4 = typename Vec4<T>::type;
  constexpr int NTW = L::NTW, LDK = L::LDK, LDC = L::LDC, LDF = L::LDF;
  constexpr int KT = DK / 16;  // key-dim tiles of the state

  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  T* sK = reinterpret_cast<T*>(smem + L::oK);
  T* sW = reinterpret_cast<T*>(smem + L::oK);
  T* sQ = reinterpret_cast<T*>(smem + L::oQ);
  T* sKT = reinterpret_cast<T*>(smem + L::oKT);
  T* sVT = reinterpret_cast<T*>(smem + L::oVT);
  T* sTw = reinterpret_cast<T*>(smem + L::oTw);
  T* sTu = reinterpret_cast<T*>(smem + L::oTu);
  T* sP = reinterpret_cast<T*>(smem + L::oP);
  float* sA = reinterpret_cast<float*>(smem + L::oA);
  float* sT = reinterpret_cast<float*>(smem + L::oT);
  float* sGl = reinterpret_cast<float*>(smem + L::oV);  // G * log2(e)
  float* seG = sGl + C;                                 // exp(G)
  float* segl = seG + C;                                // exp(G_C - G)
  float* sb = segl + C;                                 // beta
  float* sbg = sb + C;                                  // beta exp(G)

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
  const T* kgp = static_cast<const T*>(p.k);
  const T* vg = static_cast<const T*>(p.v);
  T* og = static_cast<T*>(p.o);
  const size_t qk_tok = static_cast<size_t>(p.Hqk) * DK;  // token stride of q, k
  const size_t v_tok = static_cast<size_t>(p.Hv) * DV;    // token stride of v, o

  ChunkRegs<T, DK, BV> pre;
  auto issue_loads = [&](int cs) {
    const size_t tq = static_cast<size_t>(cs) * qk_tok + static_cast<size_t>(hq) * DK;
    const size_t tv = static_cast<size_t>(cs) * v_tok + static_cast<size_t>(h) * DV + col0;
    const size_t tg = static_cast<size_t>(cs) * p.Hv + h;
    pre.load(kgp + tq, qg + tq, vg + tv, qk_tok, v_tok, p.g + tg, p.beta + tg, p.Hv, min(C, eos - cs), tid);
  };
  if (bos < eos) issue_loads(bos);

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

    // ---------------- phase 0: this chunk's operands into LDS; next chunk's loads issued ----------------
    pre.store(sK, sKT, sQ, sVT, LDK, LDC, tid);
    if (wave == 0) {
      // inclusive prefix sum of the log-gates over the chunk (G restarts every chunk)
      float G = pre.g;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(G, off);
        if (lane >= off) G += y;
      }
      const float Gl = G * kLog2e;
      const float GlC = __shfl(Gl, 63);
      const float eG = __builtin_amdgcn_exp2f(Gl);
      sGl[lane] = Gl;
      seG[lane] = eG;
      segl[lane] = __builtin_amdgcn_exp2f(GlC - Gl);
      sb[lane] = pre.b;
      sbg[lane] = pre.b * eG;
    }
    if (cs + C < eos) issue_loads(cs + C);  // lands while this chunk computes
    lds_barrier();

    // ---------------- phase 1: K K^T and Q K^T, masked with the decay ----------------
    {
      // The ten 16x16 tiles on or below the diagonal, spread over the four
      // wavefronts.  Tile (ti, tj) is computed transposed so that a lane holds
      // four consecutive columns j = 16tj + 4lg + s of row i = 16ti + lr.
      int ti[3], tj[3], nt;
      switch (wave) {
        case 0: ti[0] = 0; tj[0] = 0; ti[1] = 1; tj[1] = 0; ti[2] = 3; tj[2] = 3; nt = 3; break;
        case 1: ti[0] = 1; tj[0] = 1; ti[1] = 2; tj[1] = 0; ti[2] = 3; tj[2] = 2; nt = 3; break;
        case 2: ti[0] = 2; tj[0] = 1; ti[1] = 3; tj[1] = 0; ti[2] = 0; tj[2] = 0; nt = 2; break;
        default: ti[0] = 2; tj[0] = 2; ti[1] = 3; tj[1] = 1; ti[2] = 0; tj[2] = 0; nt = 2; break;
      }
      floatx4 kk[3], qk[3];
#pragma unroll
      for (int t = 0; t < 3; ++t) kk[t] = qk[t] = zero4();
#pragma unroll
      for (int kgi = 0; kgi < DK / MM::KG; ++kgi) {
#pragma unroll
        for (int t = 0; t < 3; ++t) {
          if (t < nt) {
            const frag a = lds_frag(sK + (16 * tj[t] + lr) * LDK, kgi, lane);
            MM::mma(kk[t], a, lds_frag(sK + (16 * ti[t] + lr) * LDK, kgi, lane));
            MM::mma(qk[t], a, lds_frag(sQ + (16 * ti[t] + lr) * LDK, kgi, lane));
          }
        }
      }
#pragma unroll
      for (int t = 0; t < 3; ++t) {
        if (t < nt) {
          const int i = 16 * ti[t] + lr;
          const float Gi = sGl[i], bi = sb[i];
          floatx4 av = zero4(), pv = zero4();
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const int j = 16 * tj[t] + 4 * lg + s;
            if (j <= i) {  // exp(G_i - G_j) is formed only on and below the diagonal
              const float d = __builtin_amdgcn_exp2f(Gi - sGl[j]);
              av[s] = (j < i) ? bi * d * kk[t][s] : 0.f;
              pv[s] = d * qk[t][s];
            }
          }
          *reinterpret_cast<floatx4*>(sA + i * LDF + 16 * tj[t] + 4 * lg) = av;
          *reinterpret_cast<V4*>(sP + i * LDC + MM::phys_k(16 * tj[t] + 4 * lg)) =
              pack4<T>(pv[0], pv[1], pv[2], pv[3]);
        }
      }
      // zero the six tiles of P above the diagonal
      if (wave >= 2) {
#pragma unroll
        for (int t = 0; t < 3; ++t) {
          const int zi = (wave == 2) ? 0 : (t == 2 ? 2 : 1);
          const int zj = (wave == 2) ? t + 1 : (t == 2 ? 3 : t + 2);
          *reinterpret_cast<V4*>(sP + (16 * zi + lr) * LDC + MM::phys_k(16 * zj + 4 * lg)) =
              pack4<T>(0.f, 0.f, 0.f, 0.f);
        }
      }
    }
    lds_barrier();

    // ---------------- phase 2: diagonal 16x16 blocks of (I + A)^-1 ----------------
    if (wave == 0) {
      // Lane (blk, cc) computes column cc of the inverse of diagonal block blk by
      // forward substitution, x_i = [i == cc] - sum_{j < i} A_ij x_j, then stores
      // it row-major into sT and as row cc of the block's transpose into sA
      // (that block of A is not needed any more).
      const int blk = lg, cc = lr;
      const float* Ab = sA + (16 * blk) * LDF + 16 * blk;
      float x[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float arow[16];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const floatx4 a4 = *reinterpret_cast<const floatx4*>(Ab + i * LDF + 4 * q4);
          arow[4 * q4] = a4[0];
          arow[4 * q4 + 1] = a4[1];
          arow[4 * q4 + 2] = a4[2];
          arow[4 * q4 + 3] = a4[3];
        }
        float acc = (i == cc) ? 1.f : 0.f;
#pragma unroll
        for (int j = 0; j < i; ++j) acc -= arow[j] * x[j];
        x[i] = acc;
      }
      float* Tb = sT + (16 * blk) * LDF + 16 * blk;
#pragma unroll
      for (int i = 0; i < 16; ++i) Tb[i * LDF + cc] = x[i];
      float* TTb = sA + (16 * blk + cc) * LDF + 16 * blk;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *reinterpret_cast<floatx4*>(TTb + 4 * q4) = floatx4{x[4 * q4], x[4 * q4 + 1], x[4 * q4 + 2], x[4 * q4 + 3]};
    }
    lds_barrier();

    // ---------------- phase 3: off-diagonal blocks, one block diagonal at a time ----------------
    // T_ij = -T_ii * sum_{m=j}^{i-1} A_im T_mj   (16x16 blocks, i > j).  The
    // T_mj operands are read from the transposed copy above the diagonal of sA.
#pragma unroll
    for (int d = 1; d < 4; ++d) {
      if (wave < 4 - d) {
        const int bj = wave, bi = wave + d;
        floatx4 y[3];
#pragma unroll
        for (int u = 0; u < 3; ++u) {
          y[u] = zero4();
          if (u < d) {
            const int m = bj + u;
            const floatx4 af = *reinterpret_cast<const floatx4*>(sA + (16 * bi + lr) * LDF + 16 * m + 4 * lg);
            const floatx4 bf = *reinterpret_cast<const floatx4*>(sA + (16 * bj + lr) * LDF + 16 * m + 4 * lg);
            Mma<float>::mma(y[u], af, bf);
          }
        }
        const floatx4 ysum = y[0] + y[1] + y[2];
        const floatx4 tf = *reinterpret_cast<const floatx4*>(sT + (16 * bi + lr) * LDF + 16 * bi + 4 * lg);
        floatx4 t = zero4();
        Mma<float>::mma(t, tf, ysum);
        // lane holds T_ij[4lg + s][lr]
#pragma unroll
        for (int s = 0; s < 4; ++s) sT[(16 * bi + 4 * lg + s) * LDF + 16 * bj + lr] = -t[s];
        *reinterpret_cast<floatx4*>(sA + (16 * bj + lr) * LDF + 16 * bi + 4 * lg) = -t;
      }
      lds_barrier();
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
    lds_barrier();

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
    lds_barrier();

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
    lds_barrier();  // the next chunk overwrites every LDS tile
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

// Chunked-parallel prefill of the gated delta rule on gfx950.
//
// Method: the recurrence from the podcast transcript on "On the Design of
// Qwen3.8-Next Architecture", cue 14 (decay the whole state, read what the key
// holds, write only the error), in the stored layout M = S^T (dk x dv).  Inside
// a chunk of C = 64 tokens that starts from state M, unrolling the recurrence
// gives (G = inclusive in-chunk cumsum of g = log alpha):
//   A   = strict_lower(beta_i exp(G_i - G_j) (K K^T)_ij)                 (C x C)
//   (I + A) U = Z,  Z = diag(beta) (V - diag(exp G) K M)                  (C x dv)
//   O   = scale (diag(exp G) Q M + lower_incl(exp(G_i - G_j) (Q K^T)_ij) U)
//   M  <- exp(G_C) M + K^T diag(exp(G_C - G)) U
// which is exact in real arithmetic (the UT/WY form of the chunk: with
// T = (I + A)^-1, U = T diag(beta) V - T diag(beta exp G) K M).
//
// Kernel structure.  One workgroup owns one (sequence, value head, dv-slice)
// and walks its chunks in order, holding the fp32 state slice in registers the
// whole time: the state never touches HBM between chunks and no workspace
// exists.  The workgroup has eight wavefronts in two roles that run on
// different chunks at the same time:
//   producers (waves 0-3) prepare chunk n+1 into one half of a double-buffered
//     LDS stage: K (rows), K^T, V^T, the gates, the Gram products K K^T and
//     Q K^T masked with the decay (-A below the diagonal blocks, without the
//     row factor beta, and P on and below the diagonal), and the inverses
//     T_bb of the four 16x16 diagonal blocks of I + A, times diag(beta_b);
//   consumers (waves 4-7) run chunk n from the other half, each on its own
//     16-column tiles of the state: Y = K M, Z' = V - exp(G) Y, the block
//     forward substitution U_b = T_bb diag(beta_b) (Z'_b - sum_{m<b} A~_bm U_m)
//     (A_bm = diag(beta_b) A~_bm, so this is T_bb (Z_b - sum A_bm U_m) with
//     Z = diag(beta) Z'), the output tile O^T, and the state update.
// Each chunk takes three segments separated by workgroup barriers that order
// LDS only, so the producers' global loads, issued a chunk ahead, stay in
// flight.  P, -A and the block inverses are single-buffered: producers write
// chunk n+1's copies only after the consumers have used chunk n's.
//
// Matrix cores: bf16 inputs use v_mfma_f32_16x16x32_bf16 (K = 16 blocks:
// v_mfma_f32_16x16x16_bf16) with fp32 accumulation; the state, Z and U are
// rounded to bf16 only as operands.  fp32 inputs use v_mfma_f32_16x16x4_f32
// so that nothing is rounded below fp32, and run the two roles one after the
// other (the fp32 stage does not fit twice in LDS).  Accumulators feed the next
// product straight from registers (see device_common.hpp).  Decay factors are
// exp2 of log2(e)-scaled prefix sums; exp(G_i - G_j) is formed only for i >= j.
#include <atomic>
#include <type_traits>
#include <utility>

#include "device_common.hpp"
#include "launch.hpp"

namespace gdn {
namespace {

constexpr int C = 64;                    // chunk length
constexpr int NP = 4;                    // producer wavefronts (consumer wavefronts: a template parameter)
constexpr int PTHREADS = 64 * NP;
// The bf16 V tile is read only down its columns; it stores the 16-column
// blocks of a row at swizzled places: block b of row r sits at block
// b ^ swz(r).  A transposing read covers four rows of one block per 16-lane
// group and eight rows per 32 lanes; the swizzle puts those eight rows'
// 32-byte runs on eight different bank windows (unswizzled, 256-byte rows
// would put them all on the same one).
template <int W>
__device__ __forceinline__ int swz(int r) {
  constexpr int NB = W / 16;                    // 16-column blocks per row
  constexpr int RPW = W >= 128 ? 1 : 128 / W;   // rows per 256 bytes
  return (r / RPW) & (NB - 1);
}
template <int W>
__device__ __forceinline__ int swz_off(int r, int c) {  // element offset of column c of row r
  return r * W + ((((c >> 4) ^ swz<W>(r)) << 4) | (c & 15));
}
// The output tile's staging layout for 128-column bf16 tiles: 16-byte piece p of row r at p ^ (r & 15),
// so that the 16 rows one accumulator store covers, and the 16 pieces one row read covers, fall on
// distinct 16-byte bank windows.  Other tiles keep the V tile's layout.
template <class T, int W>
__device__ __forceinline__ int o_off(int r, int c) {
  if constexpr (sizeof(T) == 2 && W == 128) return r * W + ((((c >> 3) ^ (r & 15)) << 3) | (c & 7));
  else if constexpr (sizeof(T) == 2) return swz_off<W>(r, c);
  else return r * W + c;
}
// Transposing 8-byte LDS read (see lds_col4).
__device__ __forceinline__ bf16x4 tr_read(const bf16* ptr) {
  typedef short s4 __attribute__((ext_vector_type(4)));
  const s4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      reinterpret_cast<__attribute__((address_space(3))) s4*>(reinterpret_cast<size_t>(ptr)));
  return __builtin_bit_cast(bf16x4, v);
}
// lds_col4<bf16> for a swizzled tile of width W.
template <int W>
__device__ __forceinline__ bf16x4 swz_col4(const bf16* base, int r0, int c0, int lane) {
  const int lg = lane >> 4, lr = lane & 15;
  return tr_read(base + swz_off<W>(r0 + 4 * lg + (lr >> 2), c0 + 4 * (lr & 3)));
}

// The second, column-read copy of K (bf16, rows of DK keys).  The K^T operand
// for state tile a (keys per state_row) takes from each token row the four
// 8-byte runs of keys 32(a>>1) + 4(a&1) + 8m, m = 0..3, 16 bytes apart.  The
// 8-byte units u of row r are stored at u ^ (8 kn_x(r) + kn_e(r)): kn_x
// permutes pairs of 32-byte blocks and kn_e swaps the halves of each 16-byte
// piece, so the eight rows one 32-lane half of a transposing read covers use
// 32 distinct bank pairs.  kn_e is bit 2 of the row.
template <int DK>
__device__ __forceinline__ int kn_x(int r) { return (r / (128 / DK)) & (DK / 32 - 1); }
__device__ __forceinline__ int kn_e(int r) { return (r >> 2) & 1; }
// Element offset of the (unswapped) 16-byte piece pc of row r.
template <int DK>
__device__ __forceinline__ int kn_piece(int r, int pc) { return r * DK + 8 * (pc ^ (kn_x<DK>(r) << 2)); }
// Read addresses, split into a per-lane part and a per-tile part: the rows a
// transposing read covers start at multiples of 8, where the swizzle depends
// on the lane only.
template <int DK>
struct KnCols {
  const bf16* lane_base;
  int x, e;
  __device__ __forceinline__ KnCols(const bf16* base, int lane) {
    const int rl = 4 * (lane >> 4) + ((lane & 15) >> 2);
    x = kn_x<DK>(rl);
    e = kn_e(rl);
    lane_base = base + rl * DK + 8 * (lane & 3);
  }
  __device__ __forceinline__ const bf16* tile(int a) const {
    return lane_base + 32 * ((a >> 1) ^ x) + 4 * ((a & 1) ^ e);
  }
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

// Per-token gate vectors of a chunk, C floats each, in this order.
enum { VEC_EG, VEC_BETA, VEC_EGC_G, VEC_EGC, VEC_GL, VEC_E0, VEC_N = VEC_E0 + 3 };

// Decay factors exp(G_i - G_j) (j <= i, else 0) of the 16x16 tile (ti, tj) of a
// chunk, for the accumulator layout that gives the lane i = 16ti + lr and
// j = 16tj + 4lg + s.  Below the diagonal blocks they are products of two
// factors no larger than one that the gate scan stores, exp(G_i - G_r) and
// exp(G_r - G_j) with r the last token of tile tj (G is non-increasing);
// on a diagonal block they are formed directly.
__device__ __forceinline__ floatx4 decay_tile(const float* vec, int ti, int tj, int lg, int lr) {
  const int i = 16 * ti + lr;
  floatx4 d;
  if (ti > tj) {
    const float* e = vec + (VEC_E0 + tj) * C;
    const floatx4 ej = *reinterpret_cast<const floatx4*>(e + 16 * tj + 4 * lg);
    d = ej * e[i];
  } else {
    const float* gl = vec + VEC_GL * C;
    const float Gi = gl[i];
    const floatx4 Gj = *reinterpret_cast<const floatx4*>(gl + 16 * tj + 4 * lg);
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const int j = 16 * tj + 4 * lg + s4;
      d[s4] = __builtin_amdgcn_exp2f(j <= i ? Gi - Gj[s4] : -__builtin_inff());  // exp2(-inf) = 0
    }
  }
  return d;
}

// LDS layout.  K and Q rows are padded against bank conflicts (see LDK).
template <class T, int DK, int BV, int NSTAGE, int NCW, bool OUTW>
struct Layout {
  static constexpr int EPB = 16 / sizeof(T);
  static constexpr int NTW = BV / (16 * NCW);   // 16-column state tiles per consumer wave
  // [C][DK] rows of K and Q (natural key order), padded so that the 16 rows
  // one 16-byte row read covers fall on distinct banks: bf16 rows take 32
  // bytes of padding (16 bytes leave a two-way conflict on gfx950).  fp32
  // keeps 16, which also serves its column reads.
  static constexpr int LDK = DK + (sizeof(T) == 2 ? 2 * EPB : EPB);
  static constexpr int LDV = BV;                // [C][BV] rows: V (only read down its columns; bf16 swizzled)
  // bf16 keeps a second copy of K for the transposing reads of K^T, swizzled
  // for them (kn_piece); out of the padded rows they would conflict on banks.
  static constexpr bool KNAT = sizeof(T) == 2;
  static constexpr int KGC = C / Mma<T>::KG;    // k-groups over the chunk
  static constexpr int LDA = 20;                // fp32 diagonal blocks of A
  // one stage, double-buffered: written by the producers in segment 1
  static constexpr size_t sK = 0;
  static constexpr size_t sQ = sK + sizeof(T) * C * LDK;
  static constexpr size_t sV = sQ + sizeof(T) * C * LDK;
  static constexpr size_t sKn = sV + sizeof(T) * C * LDV;   // [C][DK] K, column-read copy (bf16)
  // per-token vectors (VEC_*): exp G, beta, exp(G_C - G) (the first and third
  // with the state's carried scale folded in), the state's factor and scale
  // (VEC_EGC lanes 0 and 1), G log2(e), and the decay to or from the last token
  // of 16-token tiles 0-2
  static constexpr size_t sVec = sKn + (KNAT ? sizeof(T) * C * DK : 0);
  static constexpr size_t stage_bytes = (sVec + VEC_N * 4 * C + 15) / 16 * 16;
  // Single-buffered, written by the producers in segment 1 after the
  // consumers have read the previous chunk's copy in segment 2.  All three
  // are kept in "fragment order": the 16 (or 8) bytes one lane contributes to
  // a matrix-core operand are stored contiguously, lane after lane, so both
  // the producers' writes and the consumers' reads are conflict-free.
  //   P:   per (token tile ct, k-group kg), the B operand P^T of O^T += U^T P^T
  //        (with output waves written by them, in segment 2)
  //   -A:  the A operands of the block substitution: (1,0); (2,0)+(2,1); (3,0)+(3,1); (3,2)
  //   T_bb: the A operands (I + A_bb)^-1 of the four diagonal blocks
  static constexpr size_t oPf = NSTAGE * stage_bytes;
  static constexpr size_t oAnf = oPf + size_t(4) * KGC * 64 * 16;
  static constexpr size_t oTbf = oAnf + size_t(6) * 64 * 4 * sizeof(T);
  // producer scratch
  static constexpr size_t oAd = oTbf + size_t(4) * 64 * 4 * sizeof(T);
  // With output wavefronts: the state and U of each consumer wave as bf16
  // matrix-core operands, fragment order (the state written in segment 3 for
  // the next chunk, U in segment 2; read by the paired output wave in
  // segments 1 and 3).
  static constexpr size_t oMx = oAd + 4 * 4 * 16 * LDA;
  static constexpr size_t oUx = oMx + (OUTW ? size_t(NCW) * (DK / Mma<T>::KG) * 64 * 16 : 0);
  static constexpr size_t bytes = oUx + (OUTW ? size_t(NCW) * KGC * 64 * 16 : 0);
  static_assert(!OUTW || NTW == 1, "output wavefronts pair with one-tile consumer waves");
  static_assert(BV % (16 * NCW) == 0, "every consumer wave owns whole 16-column tiles");
  static_assert(sQ % 16 == 0 && sV % 16 == 0 && sKn % 16 == 0 && sVec % 16 == 0 && oPf % 16 == 0 &&
                oAnf % 16 == 0 && oTbf % 16 == 0 && oAd % 16 == 0 && oMx % 16 == 0 && oUx % 16 == 0,
                "16-byte aligned LDS regions");
  // element offsets into the fragment-order buffers
  // P: tile (ti, tj) of the lane's piece (4 elements) inside fragment (ti, tj / TPG)
  __device__ __forceinline__ static int pf(int ti, int tj, int lane) {
    constexpr int TPG = Mma<T>::TPG, FE = 16 / sizeof(T);
    return ((ti * KGC + tj / TPG) * 64 + lane) * FE + (tj % TPG) * 4;
  }
  // -A: bf16 pairs the tiles (b,0) and (b,1) of b = 2, 3 into one 32-wide fragment
  __device__ __forceinline__ static int anf(int ti, int tj, int lane) {
    if constexpr (Mma<T>::TPG == 2) {
      if (ti == 1) return lane * 4;                              // (1,0)
      if (tj < 2) return 256 + (ti - 2) * 512 + lane * 8 + tj * 4;  // (2,0) (2,1) (3,0) (3,1)
      return 1280 + lane * 4;                                    // (3,2)
    } else {
      const int k = ti == 1 ? 0 : (ti == 2 ? 1 + tj : 3 + tj);   // (1,0) (2,0) (2,1) (3,0) (3,1) (3,2)
      return (k * 64 + lane) * 4;
    }
  }
  __device__ __forceinline__ static int tbf(int b, int lane) { return (b * 64 + lane) * 4; }
};

struct Params {
  const void *q, *k, *v;
  const float *g, *beta, *h0;
  const int32_t* cu;
  void* o;
  float* hT;
  void *save_state, *save_u;  // element type T
  const int32_t* chunk_base;
  const int32_t* order;  // packed sequences, longest first (null: natural order)
  // SEG: segments of seg_len tokens (see seg.hip); qt receives the transition
  // runs' outputs, seg_fin / seg_phi their end states [nseg][batch][Hv][DK][DV]
  void* qt;
  float *seg_fin, *seg_phi;
  int seg_len, nseg, batch;
  int T, Hqk, Hv, nslices;
  int grp, ngroups;  // units per group sharing keys and queries, number of groups
  float scale;
};

// Producers' raw operands of one chunk (K rows, this slice's V rows, gates),
// loaded one chunk ahead.
template <class T, int DK, int BV>
struct ChunkRegs {
  typedef typename Mma<T>::frag frag;
  static constexpr int EPB = 16 / sizeof(T);
  static constexpr int KPR = DK / EPB;                  // 16-byte pieces per K / Q row
  static constexpr int KIT = C * KPR / PTHREADS;        // K (and Q) pieces per producer thread
  static constexpr int RPI = 64 / KPR;                  // K rows per wave-wide load
  static constexpr int VPR = BV / EPB;                  // 16-byte pieces per V row (this slice)
  static constexpr int VIT = (C * VPR + PTHREADS - 1) / PTHREADS;
  static_assert(C * KPR % PTHREADS == 0 && KIT % 2 == 0 && RPI % 4 == 0, "K rows split evenly");
  frag k[KIT], q[KIT], v[VIT];
  float g, b;

  // Row of the K / Q piece a producer thread holds in slot it (its column is
  // piece lane % KPR).  Bit 2 of the row is bit 0 of it, so the half swap of
  // the column-read K copy (kn_e) is known at compile time.
  __device__ __forceinline__ static int kq_row(int it, int tid) {
    const int rr = (tid & 63) / KPR, w = tid >> 6;
    return (rr & 3) | ((it & 1) << 2) | (((rr >> 2) + (RPI / 4) * (w + NP * (it >> 1))) << 3);
  }

  // Every load is unconditional and reads a valid row (rows past the end of
  // the sequence read its last token): a select on a loaded value would make
  // the compiler wait for the load on the spot.  The padded rows are finite
  // and harmless because their gates are masked to g = 0, beta = 0, which
  // zeroes their rows of A, Z and U exactly.  Consecutive lanes read
  // consecutive 16-byte pieces of a row.
  // Offsets inside a chunk are 32-bit byte counts (a token row of q, k or v
  // is at most 4096 heads x 128 x 4 bytes, checked on the host), so the
  // loads take a uniform 64-bit base plus one 24-bit multiply per row.
  __device__ __forceinline__ void load(const T* kb, const T* qb, const T* vb, uint32_t qk_row, uint32_t v_row,
                                       const float* gb, const float* bb, uint32_t g_row, int Lc, int tid,
                                       bool vzero = false) {
    const char* kc = reinterpret_cast<const char*>(kb);
    const char* qc = reinterpret_cast<const char*>(qb);
    const char* vc = reinterpret_cast<const char*>(vb);
#pragma unroll
    for (int it = 0; it < KIT; ++it) {
      const uint32_t off = __umul24(min(kq_row(it, tid), Lc - 1), qk_row) + (tid % KPR) * 16;
      k[it] = *reinterpret_cast<const frag*>(kc + off);
      q[it] = *reinterpret_cast<const frag*>(qc + off);
    }
    if (vzero) {  // (a workgroup-uniform branch)
#pragma unroll
      for (int it = 0; it < VIT; ++it) v[it] = frag{};
    } else {
#pragma unroll
      for (int it = 0; it < VIT; ++it) {
        const int t = min(tid + it * PTHREADS, C * VPR - 1);
        v[it] = *reinterpret_cast<const frag*>(vc + __umul24(min(t / VPR, Lc - 1), v_row) + (t % VPR) * 16);
      }
    }
    const int gl = tid - (PTHREADS - 64);  // the last producer wave owns the gates, one token per lane
    if (gl >= 0) {
      const uint32_t off = __umul24(min(gl, Lc - 1), g_row);
      g = *reinterpret_cast<const float*>(reinterpret_cast<const char*>(gb) + off);
      b = *reinterpret_cast<const float*>(reinterpret_cast<const char*>(bb) + off);
    }
  }

  // K, Q -> padded rows in natural key order; V and (if sKn) the column-read
  // copy of K -> swizzled rows.  Every store is one 16-byte piece.
  __device__ __forceinline__ void store(T* sK, T* sQ, T* sV, T* sKn, int LDK, int LDV, int tid) const {
#pragma unroll
    for (int it = 0; it < KIT; ++it) {
      const int r = kq_row(it, tid), pc = tid % KPR;
      *reinterpret_cast<frag*>(sK + r * LDK + pc * EPB) = k[it];
      *reinterpret_cast<frag*>(sQ + r * LDK + pc * EPB) = q[it];
      if constexpr (sizeof(T) == 2) {
        if (sKn) {
          const frag x = (it & 1) ? __builtin_shufflevector(k[it], k[it], 4, 5, 6, 7, 0, 1, 2, 3) : k[it];
          *reinterpret_cast<frag*>(sKn + kn_piece<DK>(r, pc)) = x;
        }
      }
    }
#pragma unroll
    for (int it = 0; it < VIT; ++it) {
      const int t = tid + it * PTHREADS;
      if (t < C * VPR) {
        const int r = t / VPR, c = (t % VPR) * EPB;
        *reinterpret_cast<frag*>(sV + (sizeof(T) == 2 ? swz_off<BV>(r, c) : r * LDV + c)) = v[it];
      }
    }
  }
};

// Gram tiles (ti >= tj) of producer wave W, grouped by token-row tile so that
// a wave loads each B fragment (K and Q rows of tile ti) once per k-group.
// Every tile gives A; P comes from Q K^T of the same tiles, except with two
// output waves, which form P themselves but for the tiles in pmask (bit t:
// tile t), the tiles (2,0) and (3,3) in either assignment.
// With output waves (ROWS = false):
//   wave 0: (3,0) (3,1) (3,2)    wave 1: (2,0) (2,1)
//   wave 2: (1,0) (1,1) (2,2)    wave 3: (0,0) (3,3)
// Without (ROWS = true), by token-row block, which needs 15 distinct row
// fragments per k-group over the four waves instead of 18 (0.7-2 % faster on
// the 128-column shapes, 1 % slower with output waves):
//   wave 0: (0,0) (1,0) (1,1)    wave 1: (2,0) (2,1) (2,2)
//   wave 2: (3,0) (3,1)          wave 3: (3,2) (3,3)
template <int W, bool ROWS> struct GramTiles;
template <> struct GramTiles<0, false> { static constexpr int n = 3, ti[3] = {3, 3, 3}, tj[3] = {0, 1, 2}, pmask = 0; };
template <> struct GramTiles<1, false> { static constexpr int n = 2, ti[3] = {2, 2, 0}, tj[3] = {0, 1, 0}, pmask = 1; };
template <> struct GramTiles<2, false> { static constexpr int n = 3, ti[3] = {1, 1, 2}, tj[3] = {0, 1, 2}, pmask = 0; };
template <> struct GramTiles<3, false> { static constexpr int n = 2, ti[3] = {0, 3, 0}, tj[3] = {0, 3, 0}, pmask = 2; };
template <> struct GramTiles<0, true> { static constexpr int n = 3, ti[3] = {0, 1, 1}, tj[3] = {0, 0, 1}, pmask = 0; };
template <> struct GramTiles<1, true> { static constexpr int n = 3, ti[3] = {2, 2, 2}, tj[3] = {0, 1, 2}, pmask = 1; };
template <> struct GramTiles<2, true> { static constexpr int n = 2, ti[3] = {3, 3, 0}, tj[3] = {0, 1, 0}, pmask = 0; };
template <> struct GramTiles<3, true> { static constexpr int n = 2, ti[3] = {3, 3, 0}, tj[3] = {2, 3, 0}, pmask = 2; };

// P tiles (ti >= tj) formed by output wave W (with two output waves only):
// the eight the producers leave.
template <int W> struct OutPTiles;
template <> struct OutPTiles<0> { static constexpr int n = 4, ti[4] = {0, 1, 1, 3}, tj[4] = {0, 0, 1, 0}; };
template <> struct OutPTiles<1> { static constexpr int n = 4, ti[4] = {2, 2, 3, 3}, tj[4] = {1, 2, 1, 2}; };

// SAVE: the variant a backward pass runs first; it keeps each chunk's starting
// state and U (as T, the precision of the products' operands) and writes no
// output.  SEG: the segmented variant (seg.hip): the units are virtual
// sequences, a segment of a batch row each.
template <class T, int DK, int DV, int BV, int NSTAGE, int NCW, bool OUTW, bool SAVE, bool SEG>
__global__ __launch_bounds__(64 * (NP + NCW * (OUTW ? 2 : 1))) void prefill_kernel(Params p) {
  using L = Layout<T, DK, BV, NSTAGE, NCW, OUTW>;
  using MM = Mma<T>;
  using M16 = Mma16<T>;
  using frag = typename MM::frag;
  using V4 = typename Vec4<T>::type;
  constexpr int NTW = L::NTW, LDK = L::LDK, LDV = L::LDV, LDA = L::LDA;
  constexpr int KT = DK / 16;       // key-dim tiles of the state
  constexpr int KGK = DK / MM::KG;  // k-groups over the key dim
  constexpr int KGC = C / MM::KG;   // k-groups over the chunk

  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  float* sAd = reinterpret_cast<float*>(smem + L::oAd);  // [4][16][LDA] fp32 diagonal blocks of A, transposed

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const bool producer = wave < NP;
  const bool consumer = !producer && wave < NP + NCW;  // else (OUTW) an output wave
  const int lg = lane >> 4;
  const int lr = lane & 15;

  // Workgroup -> (unit, dv-slice).  Units that read the same keys and queries
  // (the value heads of one q/k head; in the segmented variant also the
  // zero-state and transition runs of one segment) form a group of p.grp, and
  // the members of a group and their slices get ids 8 apart, so they run on
  // one XCD and share its L2.
  const int xcd = blockIdx.x & 7;
  const int rest = blockIdx.x >> 3;
  const int slice = rest % p.nslices;
  const int member = (rest / p.nslices) % p.grp;
  const int grp = (rest / p.nslices / p.grp) * 8 + xcd;
  if (grp >= p.ngroups) return;
  const int hg = p.Hv / p.Hqk;  // value heads per q/k head
  int n, h;
  int b, seg = 0;    // SEG: the batch row and segment of the run
  bool phi = false;  // SEG: a transition run (v = 0 from the identity state)
  int bos, eos;
  if constexpr (SEG) {
    // group (row, segment, q/k head); member (run, value head): segment 0 has
    // one run from the row's initial state, every later segment a run from the
    // zero state and a transition run
    const int bs = grp / p.Hqk, run = member / hg;
    seg = bs % p.nseg;
    b = bs / p.nseg;
    if (seg == 0 && run > 0) return;
    h = (grp % p.Hqk) * hg + member % hg;
    phi = run == 1;
    n = seg == 0 ? b : p.batch + b * 2 * (p.nseg - 1) + 2 * (seg - 1) + run;  // (virtual sequence)
    bos = b * p.T + seg * p.seg_len;
    eos = min(b * p.T + p.T, bos + p.seg_len);
  } else {
    const int unit = grp * p.grp + member;  // = sequence * Hv + h
    h = unit % p.Hv;
    n = p.order ? p.order[unit / p.Hv] : unit / p.Hv;
    b = n;
    bos = p.cu ? p.cu[n] : n * p.T;
    eos = p.cu ? p.cu[n + 1] : bos + p.T;
  }
  const int hq = h / hg;
  const int nch = (eos - bos + C - 1) / C;
  const int col0 = slice * BV;
  const int cw = producer ? 0 : (wave - NP) % NCW;  // consumer index (an output wave: its consumer's)
  const int wcol = col0 + cw * 16 * NTW;             // first state column of a consumer (or output) wave

  const T* qg = static_cast<const T*>(p.q);
  const T* kgp = static_cast<const T*>(p.k);
  const T* vg = static_cast<const T*>(p.v);
  T* og = static_cast<T*>(SEG && phi ? p.qt : p.o);
  const size_t qk_tok = static_cast<size_t>(p.Hqk) * DK;
  const size_t v_tok = static_cast<size_t>(p.Hv) * DV;

  auto stage = [&](int s) __attribute__((always_inline)) { return smem + s * L::stage_bytes; };

  // ------------------------------------------------------------ producer state
  ChunkRegs<T, DK, BV> pre;
  auto issue_loads = [&](int c) __attribute__((always_inline)) {
    const int cs = bos + c * C;
    const size_t tq = static_cast<size_t>(cs) * qk_tok + static_cast<size_t>(hq) * DK;
    const size_t tv = static_cast<size_t>(cs) * v_tok + static_cast<size_t>(h) * DV + col0;
    const size_t tg = static_cast<size_t>(cs) * p.Hv + h;
    pre.load(kgp + tq, qg + tq, vg + tv, static_cast<uint32_t>(qk_tok * sizeof(T)),
             static_cast<uint32_t>(v_tok * sizeof(T)), p.g + tg, p.beta + tg, static_cast<uint32_t>(p.Hv * 4),
             min(C, eos - cs), tid, SEG && phi);
  };

  // The state's decay is applied lazily (not in a saving run, whose stored
  // chunk-start states are the state itself): the consumers hold Ms with
  // M = 2^L Ms, and the gate-scan wave carries L from chunk to chunk, folding
  // 2^L into exp(G) (Y = K M and Q M read Ms) and 2^-L into U's decay before the
  // update, so that Ms' = Ms + K^T (2^(-G - L) U) needs no multiply of the
  // state; 2^L then takes the chunk's decay exp(G_C).  When L would leave
  // [-64, 64] the state is renormalised instead: Ms is multiplied by 2^(G_C + L)
  // (the eager update) and L restarts at 0.  VEC_EGC holds the state's factor
  // for the chunk (lane 0: 1, or the renormalising factor) and the scale after
  // it (lane 1), which the end-state writes apply.
  constexpr bool LAZY = !SAVE;
  float lazyL = 0.f;  // the gate-scan wave's copy of L

  // Stage the chunk's K, Q, V and gates; issue the next chunk's loads.  (The
  // loads sit in this segment because here the producers have slack: the
  // consumers' segment 2 is the longer one.)
  auto prod_stores = [&](int c, int s) __attribute__((always_inline)) {
    unsigned char* S = stage(s);
    const int cs = bos + c * C, Lc = min(C, eos - cs);
    pre.store(reinterpret_cast<T*>(S + L::sK), reinterpret_cast<T*>(S + L::sQ), reinterpret_cast<T*>(S + L::sV),
              L::KNAT ? reinterpret_cast<T*>(S + L::sKn) : nullptr, LDK, LDV, tid);
    if (wave == NP - 1) {  // the lightest producer wave in this segment and the next
      const bool live = lane < Lc;  // tokens past the end act as g = 0, beta = 0 (exact no-ops)
      const float bt = live ? pre.b : 0.f;
      // inclusive prefix sum of the log-gates over the chunk
      const float Gl = wave_inclusive_sum(live ? fmaxf(pre.g, kGateFloor) : 0.f) * kLog2e;
      const float GlC = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, Gl), 63));
      float* vec = reinterpret_cast<float*>(S + L::sVec);
      vec[VEC_BETA * C + lane] = bt;
      vec[VEC_GL * C + lane] = Gl;
      if constexpr (LAZY) {
        const float aL = GlC + lazyL;                      // log2 of the state's factor after this chunk
        const bool renorm = !(aL >= -64.f && aL <= 64.f);  // (uniform)
        const float fac = __builtin_amdgcn_exp2f(aL);
        vec[VEC_EG * C + lane] = __builtin_amdgcn_exp2f(Gl + lazyL);
        vec[VEC_EGC_G * C + lane] = __builtin_amdgcn_exp2f(renorm ? GlC - Gl : -Gl - lazyL);
        vec[VEC_EGC * C + lane] = lane == 1 ? (renorm ? 1.f : fac) : (renorm ? fac : 1.f);
        lazyL = renorm ? 0.f : aL;
      } else {
        vec[VEC_EG * C + lane] = __builtin_amdgcn_exp2f(Gl);
        vec[VEC_EGC_G * C + lane] = __builtin_amdgcn_exp2f(GlC - Gl);
        vec[VEC_EGC * C + lane] = lane == 1 ? 1.f : __builtin_amdgcn_exp2f(GlC);
      }
#pragma unroll
      for (int b = 0; b < 3; ++b) {  // exp(-|G - G_r|), r = 16b + 15
        const float Gr = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, Gl), 16 * b + 15));
        vec[(VEC_E0 + b) * C + lane] = __builtin_amdgcn_exp2f(lane <= 16 * b + 15 ? Gr - Gl : Gl - Gr);
      }
    }
    if (c + 1 < nch) issue_loads(c + 1);
  };

  // K K^T and (without output waves, which form P themselves) Q K^T tiles,
  // masked with the decay.  The diagonal blocks of A go to LDS transposed
  // (fp32, for the inverses); -A below the diagonal and P stay in registers
  // until prod_finish.
  constexpr bool PROD_P = !(OUTW && NCW == 2);  // two output waves form most of P themselves
  constexpr bool PMASK = !(OUTW && SAVE);         // a saving run with output waves forms no P (no O)
  floatx4 pkeep[3], akeep[3];
  auto gram = [&](auto wtag, int s) __attribute__((always_inline)) {
    using GT = GramTiles<decltype(wtag)::value, !OUTW>;
    const unsigned char* S = stage(s);
    const T* sK = reinterpret_cast<const T*>(S + L::sK);
    const T* sQ = reinterpret_cast<const T*>(S + L::sQ);
    const float* vec = reinterpret_cast<const float*>(S + L::sVec);
    const float* beta = vec + VEC_BETA * C;
    floatx4 kk[3], qk[3];
#pragma unroll
    for (int t = 0; t < 3; ++t) kk[t] = qk[t] = zero4();
    // All fragments are read before the first product: under the load the
    // other roles put on the LDS, a read takes hundreds of cycles, and a
    // read-then-multiply loop over the k-groups would pay that once per group.
    frag rowk[KGK][4], rowq[KGK][4];  // fragments of token-row tiles; only the ones used are loaded
#pragma unroll
    for (int kgi = 0; kgi < KGK; ++kgi)
#pragma unroll
      for (int t = 0; t < GT::n; ++t) {
        rowk[kgi][GT::ti[t]] = lds_frag(sK + (16 * GT::ti[t] + lr) * LDK, kgi, lane);
        if (PROD_P || (PMASK && (GT::pmask >> t & 1)))
          rowq[kgi][GT::ti[t]] = lds_frag(sQ + (16 * GT::ti[t] + lr) * LDK, kgi, lane);
        rowk[kgi][GT::tj[t]] = lds_frag(sK + (16 * GT::tj[t] + lr) * LDK, kgi, lane);
      }
#pragma unroll
    for (int kgi = 0; kgi < KGK; ++kgi)
#pragma unroll
      for (int t = 0; t < GT::n; ++t) {
        MM::mma(kk[t], rowk[kgi][GT::tj[t]], rowk[kgi][GT::ti[t]]);
        if (PROD_P || (PMASK && (GT::pmask >> t & 1))) MM::mma(qk[t], rowk[kgi][GT::tj[t]], rowq[kgi][GT::ti[t]]);
      }
    // lane holds X[i = 16ti + lr][j = 16tj + 4lg + s] of both products
#pragma unroll
    for (int t = 0; t < 3; ++t) {
      pkeep[t] = akeep[t] = zero4();
      if (t < GT::n) {
        const int i = 16 * GT::ti[t] + lr;
        const float bi = beta[i];
        const floatx4 dd = decay_tile(vec, GT::ti[t], GT::tj[t], lg, lr);
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
          const int j = 16 * GT::tj[t] + 4 * lg + s4;
          const float d = dd[s4];
          // The diagonal blocks keep beta (their inverses are formed from
          // them); below them A_bm = diag(beta_b) A~_bm, and the factor moves
          // onto the columns of the inverses (see prod_finish).
          if (GT::ti[t] == GT::tj[t]) akeep[t][s4] = j < i ? bi * d * kk[t][s4] : 0.f;
          else akeep[t][s4] = d * kk[t][s4];
          if (PROD_P || (PMASK && (GT::pmask >> t & 1))) pkeep[t][s4] = d * qk[t][s4];
        }
        if (GT::ti[t] == GT::tj[t]) {
#pragma unroll
          for (int s4 = 0; s4 < 4; ++s4) sAd[(GT::ti[t] * 16 + 4 * lg + s4) * LDA + lr] = akeep[t][s4];
        }
      }
    }
  };
  auto prod_gram = [&](int s) __attribute__((always_inline)) {
    switch (wave) {
      case 0: gram(std::integral_constant<int, 0>(), s); break;
      case 1: gram(std::integral_constant<int, 1>(), s); break;
      case 2: gram(std::integral_constant<int, 2>(), s); break;
      default: gram(std::integral_constant<int, 3>(), s); break;
    }
  };

  // P (without output waves) and -A into their (single) buffers; each
  // producer wave inverts one of the four diagonal blocks of I + A.
  auto put = [&](auto wtag) __attribute__((always_inline)) {
    using GT = GramTiles<decltype(wtag)::value, !OUTW>;
    T* sPf = reinterpret_cast<T*>(smem + L::oPf);
    T* sAnf = reinterpret_cast<T*>(smem + L::oAnf);
#pragma unroll
    for (int t = 0; t < GT::n; ++t) {
      if (PROD_P || (PMASK && (GT::pmask >> t & 1)))
        *reinterpret_cast<V4*>(sPf + L::pf(GT::ti[t], GT::tj[t], lane)) =
            pack4<T>(pkeep[t][0], pkeep[t][1], pkeep[t][2], pkeep[t][3]);
      if (GT::ti[t] != GT::tj[t])
        *reinterpret_cast<V4*>(sAnf + L::anf(GT::ti[t], GT::tj[t], lane)) =
            pack4_neg<T>(akeep[t][0], akeep[t][1], akeep[t][2], akeep[t][3]);
    }
  };
  auto prod_finish = [&](int s) __attribute__((always_inline)) {
    // With output waves, the inverses are the longest chain of segment 1:
    // they get the top issue priority while they run.
    if constexpr (OUTW) __builtin_amdgcn_s_setprio(3);
    switch (wave) {
      case 0: put(std::integral_constant<int, 0>()); break;
      case 1: put(std::integral_constant<int, 1>()); break;
      case 2: put(std::integral_constant<int, 2>()); break;
      default: put(std::integral_constant<int, 3>()); break;
    }
    {  // producer wave w inverts diagonal block w of I + A
      const int cc = lane >> 2, q = lane & 3;
      const float* At = sAd + wave * 16 * LDA;  // At[j][i] = A_ij of the block
      floatx4 x;
#pragma unroll
      for (int t = 0; t < 4; ++t) x[t] = (4 * q + t == cc) ? 1.f : 0.f;
      unit_lower_inverse_column(x, At, LDA, q, std::make_integer_sequence<int, 15>());
      // The consumers solve U_b = T_bb diag(beta_b) (Z'_b - sum_{m<b} A~_bm U_m)
      // with Z' = V - exp(G) K M: beta scales column cc of the inverse here,
      // once per chunk, instead of every consumer's Z.
      x *= reinterpret_cast<const float*>(stage(s) + L::sVec)[VEC_BETA * C + 16 * wave + cc];
      // T[4q + t][cc] belongs to operand lane 16 (cc / 4) + 4q + t, element cc % 4
      T* Tb = reinterpret_cast<T*>(smem + L::oTbf);
#pragma unroll
      for (int t = 0; t < 4; ++t) Tb[L::tbf(wave, 16 * (cc >> 2) + 4 * q + t) + (cc & 3)] = from_float<T>(x[t]);
    }
    if constexpr (OUTW) __builtin_amdgcn_s_setprio(1);
  };


  // ------------------------------------------------------------ consumer state
  // Ms[a][j] holds M[state_row(a, lg, s)][wcol + 16j + lr], s = 0..3.
  floatx4 Ms[KT][NTW];
  floatx4 Z[4][NTW];  // Z, then U, by 16-row token block
  frag mfr[KGK][NTW];  // the state as matrix-core operands (bf16-rounded for bf16 inputs), per chunk
  // the unit's state: uniform base, small per-lane offsets (keeps 64-bit
  // per-element addresses out of the registers)
  const size_t sbase = (static_cast<size_t>(n) * p.Hv + h) * DK * DV;
  const int slane = MM::state_row(0, lg, 0) * DV + wcol + lr;
  if (consumer) {
    if constexpr (SEG) {  // the row's initial state, the zero state, or (transition runs) the identity
      const float* h0 = seg == 0 && p.h0 ? p.h0 + (static_cast<size_t>(b) * p.Hv + h) * DK * DV : nullptr;
#pragma unroll
      for (int a = 0; a < KT; ++a)
#pragma unroll
        for (int j = 0; j < NTW; ++j)
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const int row = MM::state_row(a, lg, s), col = wcol + 16 * j + lr;
            Ms[a][j][s] = h0 ? h0[row * DV + col] : (phi && row == col ? 1.f : 0.f);
          }
    } else {
      const float* h0 = p.h0 + sbase;
#pragma unroll
      for (int a = 0; a < KT; ++a)
#pragma unroll
        for (int j = 0; j < NTW; ++j)
#pragma unroll
          for (int s = 0; s < 4; ++s) Ms[a][j][s] = p.h0 ? h0[slane + MM::state_row(a, 0, s) * DV + 16 * j] : 0.f;
    }
  }

  // The state at the start of chunk c (SAVE).
  auto save_state = [&](int c) __attribute__((always_inline)) {
    const int cb = p.chunk_base ? p.chunk_base[n] : n * ((p.T + C - 1) / C);
    T* d = static_cast<T*>(p.save_state) + (static_cast<size_t>(cb + c) * p.Hv + h) * DK * DV;
#pragma unroll
    for (int a = 0; a < KT; ++a)
#pragma unroll
      for (int j = 0; j < NTW; ++j)
#pragma unroll
        for (int s = 0; s < 4; ++s) d[slane + MM::state_row(a, 0, s) * DV + 16 * j] = from_float<T>(Ms[a][j][s]);
  };

  // seg 1: Y = K M; Z' = V - exp(G) Y (beta is applied through the inverses).  With one state tile per wave the
  // state part of the output, O^T = diag-scaled (Q M)^T, is formed here too,
  // next to K M which takes the same operands; with two, holding it until
  // seg 2 would exceed the register budget, and seg 2 forms it instead.
  constexpr bool QM_EARLY = NTW == 1 && !OUTW;
  // Where the consumers copy a chunk's output rows from LDS to HBM.  With two
  // state tiles per wave, segment 1 (K M and Z only) ends before the
  // producers' and leaves the consumers idle at its barrier, while segment 3
  // is the longest of the chunk; so the rows of chunk c go out at the end of
  // the consumers' segment 1 of chunk c + 1 (their LDS tile, in the spent V
  // tile of c's stage, is refilled only in segment 2 of chunk c + 1), and the
  // last chunk's after the loop: 4 % off the packed 64-sequence launch, 9 %
  // off the segmented long row, the same results.  With one tile per wave, segment 1 also forms (Q M)^T and has no
  // slack; the rows go out at the start of segment 3 of the same chunk.
  constexpr bool ROWS_NEXT = !OUTW && !SAVE && !QM_EARLY;
  frag* sMx = reinterpret_cast<frag*>(smem + L::oMx) + cw * KGK * 64;  // this column tile's exchange slots
  frag* sUx = reinterpret_cast<frag*>(smem + L::oUx) + cw * KGC * 64;
  // The state as matrix-core operands (bf16-rounded for bf16 inputs); with
  // output waves also handed to the paired output wave.
  auto state_operands = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int kgi = 0; kgi < KGK; ++kgi)
#pragma unroll
      for (int j = 0; j < NTW; ++j) mfr[kgi][j] = chain_frag<T>([&](int t) { return Ms[t][j]; }, kgi);
    if constexpr (OUTW) {
#pragma unroll
      for (int kgi = 0; kgi < KGK; ++kgi) sMx[kgi * 64 + lane] = mfr[kgi][0];
    }
  };
  // SAVE with output waves: the same state, from the bf16 operand copy its
  // consumer wave leaves in LDS (element e of k-group kg of lane group g is key
  // 32 kg + 8 g + e of the lane's column), and U from its copy (element e of
  // k-group kg is token 32 kg + 16 (e / 4) + 4 g + e % 4): the stores leave the
  // consumers' chain.
  auto save_state_from_operands = [&](int c) __attribute__((always_inline)) {
    const int cb = p.chunk_base ? p.chunk_base[n] : n * ((p.T + C - 1) / C);
    T* d = static_cast<T*>(p.save_state) + (static_cast<size_t>(cb + c) * p.Hv + h) * DK * DV + wcol + lr;
    if constexpr (MM::TPG == 2) {  // (output waves run with bf16 only)
#pragma unroll
      for (int kgi = 0; kgi < KGK; ++kgi) {
        const frag f = sMx[kgi * 64 + lane];
#pragma unroll
        for (int e = 0; e < 8; ++e) d[(32 * kgi + 8 * lg + e) * DV] = f[e];
      }
    }
  };
  auto save_u_from_operands = [&](int c) __attribute__((always_inline)) {
    const int cs = bos + c * C, Lc = min(C, eos - cs);
    T* u = static_cast<T*>(p.save_u) + (static_cast<size_t>(cs) * p.Hv + h) * DV + wcol + lr;
    if constexpr (MM::TPG == 2) {
#pragma unroll
      for (int kgi = 0; kgi < KGC; ++kgi) {
        const frag f = sUx[kgi * 64 + lane];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int t = 32 * kgi + 16 * (e >> 2) + 4 * lg + (e & 3);
          if (t < Lc) u[static_cast<size_t>(t) * v_tok] = f[e];
        }
      }
    }
  };

  floatx4 Ot[4][NTW];  // O^T by 16-token tile: lane holds O[16ct + lr][wcol + 16j + 4lg + s]
  auto q_times_state = [&](const T* sQ, const float* vec) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
#pragma unroll
      for (int j = 0; j < NTW; ++j) Ot[r][j] = zero4();
#pragma unroll
      for (int kgi = 0; kgi < KGK; ++kgi) {
        const frag qf = lds_frag(sQ + (16 * r + lr) * LDK, kgi, lane);
#pragma unroll
        for (int j = 0; j < NTW; ++j) MM::mma(Ot[r][j], mfr[kgi][j], qf);
      }
      const float egt = vec[VEC_EG * C + 16 * r + lr];  // exp(G) of the token this lane holds in O^T
#pragma unroll
      for (int j = 0; j < NTW; ++j) Ot[r][j] *= egt;
    }
  };
  auto cons_seg1 = [&](int s) __attribute__((always_inline)) {
    const unsigned char* S = stage(s);
    const T* sK = reinterpret_cast<const T*>(S + L::sK);
    const T* sQ = reinterpret_cast<const T*>(S + L::sQ);
    const T* sV = reinterpret_cast<const T*>(S + L::sV);
    const float* vec = reinterpret_cast<const float*>(S + L::sVec);
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int j = 0; j < NTW; ++j) Z[r][j] = zero4();
    if constexpr (!OUTW) state_operands();  // (with output waves they were formed after the last update)
#pragma unroll
    for (int kgi = 0; kgi < KGK; ++kgi) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const frag af = lds_frag(sK + (16 * r + lr) * LDK, kgi, lane);
#pragma unroll
        for (int j = 0; j < NTW; ++j) MM::mma(Z[r][j], af, mfr[kgi][j]);
      }
    }
    if constexpr (QM_EARLY) q_times_state(sQ, vec);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float eg[4];
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) eg[s4] = vec[VEC_EG * C + 16 * r + 4 * lg + s4];
#pragma unroll
      for (int j = 0; j < NTW; ++j) {
        V4 v4;
        if constexpr (sizeof(T) == 2)
          v4 = swz_col4<BV>(sV, 16 * r, (cw * NTW + j) * 16, lane);
        else
          v4 = lds_col4<T>(sV, LDV, 16 * r, (cw * NTW + j) * 16, lane);
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) Z[r][j][s4] = to_float(v4[s4]) - eg[s4] * Z[r][j][s4];  // Z' (beta is in T)
      }
    }
  };

  // O^T += U^T P^T over the chunk's token tiles, then O -> HBM (U from Z, or,
  // in an output wave, from the exchange slots).
  auto out_pu = [&](int c, int s, const frag* uex = nullptr) __attribute__((always_inline)) {
    const T* sPf = reinterpret_cast<const T*>(smem + L::oPf);
    const int cs = bos + c * C, Lc = min(C, eos - cs);
    // every P fragment read from LDS feeds all of the wave's n-tiles
#pragma unroll
    for (int kgi = 0; kgi < KGC; ++kgi) {
      frag uf[NTW];
#pragma unroll
      for (int j = 0; j < NTW; ++j)
        uf[j] = uex ? uex[kgi * 64 + lane] : chain_frag<T>([&](int t) { return Z[t][j]; }, kgi);
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        if (kgi * MM::KG <= 16 * ct + 15) {  // P is zero above the diagonal
          const frag pf = *reinterpret_cast<const frag*>(sPf + L::pf(ct, kgi * MM::TPG, lane));
#pragma unroll
          for (int j = 0; j < NTW; ++j) MM::mma(Ot[ct][j], uf[j], pf);
        }
      }
    }
    // The query scale, skipped when it is 1 (a uniform branch: the product is
    // then exact and the multiplies are spared).  Output waves multiply
    // unconditionally: there the branch measured 1 % slower.
    if constexpr (!SAVE) {
      if (OUTW || p.scale != 1.f) {
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
#pragma unroll
          for (int j = 0; j < NTW; ++j) Ot[ct][j] *= p.scale;
      }
    }
    if constexpr (SAVE) {
      (void)cs;
      (void)Lc;
    } else if constexpr (OUTW) {
      T* orow = og + static_cast<size_t>(cs + lr) * v_tok + static_cast<size_t>(h) * DV + wcol + 4 * lg;
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        if (16 * ct + lr < Lc) {
#pragma unroll
          for (int j = 0; j < NTW; ++j) {
            const floatx4 ov = Ot[ct][j];
            *reinterpret_cast<V4*>(orow + static_cast<size_t>(16 * ct) * v_tok + 16 * j) =
                pack4<T>(ov[0], ov[1], ov[2], ov[3]);
          }
        }
      }
    } else {
      // The output tile goes to LDS first, into the chunk's V tile (V is used
      // up by now and the stage is not refilled before the next chunk's
      // segment 2); o_rows_out then writes it as whole rows.  Written straight
      // from the accumulator layout, every store would cover 16 rows with 32
      // bytes each, and the memory path would stall the consumer for a large
      // part of the chunk.
      T* sO = reinterpret_cast<T*>(stage(s) + L::sV);
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int j = 0; j < NTW; ++j) {
          const floatx4 ov = Ot[ct][j];
          const int r = 16 * ct + lr, col = (cw * NTW + j) * 16 + 4 * lg;
          *reinterpret_cast<V4*>(sO + o_off<T, BV>(r, col)) = pack4<T>(ov[0], ov[1], ov[2], ov[3]);
        }
    }
  };
  // The chunk's output rows, BV columns each, from LDS to HBM in 16-byte
  // pieces (consecutive lanes cover consecutive pieces of a row).
  auto o_rows_out = [&](int c, int s) __attribute__((always_inline)) {
    constexpr int PPR = BV * sizeof(T) / 16;      // 16-byte pieces per row
    constexpr int NT = 64 * NCW;                  // consumer threads
    constexpr int EP = 16 / sizeof(T);
    constexpr int NIT = C * PPR / NT;
    static_assert(C * PPR % NT == 0, "whole passes over the tile");
    const T* sO = reinterpret_cast<const T*>(stage(s) + L::sV);
    const int cs = bos + c * C, Lc = min(C, eos - cs);
    const int ct0 = tid - 64 * NP;
    // Every row is read from LDS first (the tile holds all C rows), so the
    // stores wait for LDS once; the stores of rows past the end are skipped.
    // Addresses: the chunk's first row as a uniform base plus a 32-bit byte
    // offset per lane (C rows of one head span far less than 4 GiB).
    frag rows[NIT];
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int t = ct0 + it * NT;
      rows[it] = *reinterpret_cast<const frag*>(sO + o_off<T, BV>(t / PPR, (t % PPR) * EP));
    }
    char* obase = reinterpret_cast<char*>(og + static_cast<size_t>(cs) * v_tok + static_cast<size_t>(h) * DV + col0);
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int t = ct0 + it * NT;
      const int r = t / PPR, col = (t % PPR) * EP;
      const uint32_t off = (static_cast<uint32_t>(r) * static_cast<uint32_t>(v_tok) + col) * sizeof(T);
      if (r < Lc) *reinterpret_cast<frag*>(obase + off) = rows[it];
    }
  };

  // seg 2: U by block forward substitution; O^T += U^T P^T; O -> HBM.
  auto cons_seg2 = [&](int c, int s) __attribute__((always_inline)) {
    if constexpr (!QM_EARLY && !OUTW) {  // the state operands are formed again rather than held over the barrier
#pragma unroll
      for (int kgi = 0; kgi < KGK; ++kgi)
#pragma unroll
        for (int j = 0; j < NTW; ++j) mfr[kgi][j] = chain_frag<T>([&](int t) { return Ms[t][j]; }, kgi);
      q_times_state(reinterpret_cast<const T*>(stage(s) + L::sQ), reinterpret_cast<const float*>(stage(s) + L::sVec));
    }
    const T* sAnf = reinterpret_cast<const T*>(smem + L::oAnf);
    const T* sTbf = reinterpret_cast<const T*>(smem + L::oTbf);
    using F16 = typename M16::frag;
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
      // U_b = T_bb (Z_b + sum_{m<b} (-A_bm) U_m), b = 0..3
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        floatx4 w = Z[b][j];
        if (b >= 2) {  // blocks 0 and 1 together: one 32-wide contraction
          if constexpr (MM::KG == 32) {
            MM::mma(w, *reinterpret_cast<const frag*>(sAnf + L::anf(b, 0, lane)), MM::chain(Z[0][j], Z[1][j]));
          } else {
            MM::mma(w, *reinterpret_cast<const frag*>(sAnf + L::anf(b, 0, lane)), Mma<float>::chain(Z[0][j]));
            MM::mma(w, *reinterpret_cast<const frag*>(sAnf + L::anf(b, 1, lane)), Mma<float>::chain(Z[1][j]));
          }
        }
        if (b == 1) M16::mma(w, *reinterpret_cast<const F16*>(sAnf + L::anf(1, 0, lane)), M16::chain(Z[0][j]));
        if (b == 3) M16::mma(w, *reinterpret_cast<const F16*>(sAnf + L::anf(3, 2, lane)), M16::chain(Z[2][j]));
        floatx4 u = zero4();
        M16::mma(u, *reinterpret_cast<const F16*>(sTbf + L::tbf(b, lane)), M16::chain(w));
        Z[b][j] = u;  // Z_b is not needed any more
      }
    }
    if constexpr (SAVE && !OUTW) {  // U rows of the chunk's tokens (with output waves: theirs to store)
      const int cs = bos + c * C, Lc = min(C, eos - cs);
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = 16 * b + 4 * lg + i;
          if (t < Lc) {
            T* u = static_cast<T*>(p.save_u) + (static_cast<size_t>(cs + t) * p.Hv + h) * DV + wcol + lr;
#pragma unroll
            for (int j = 0; j < NTW; ++j) u[16 * j] = from_float<T>(Z[b][j][i]);
          }
        }
    }
    if constexpr (OUTW) {  // U as operands for the output wave
#pragma unroll
      for (int kgi = 0; kgi < KGC; ++kgi) sUx[kgi * 64 + lane] = chain_frag<T>([&](int t) { return Z[t][0]; }, kgi);
    } else {
      out_pu(c, s);
    }
  };

  // seg 3: M <- exp(G_C) M + K^T (diag(exp(G_C - G)) U).
  // The swizzled tiles' read addresses depend on the lane in a way the
  // compiler would precompute for every column block and keep live across the
  // loop; the lane index formed afresh each chunk by an opaque (volatile) pair
  // of mbcnt instructions makes it form them where they are used instead, and
  // leaves nothing lane-derived to hold across the loop.
  auto opaque_lane = [&]() __attribute__((always_inline)) {
    int v;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(v));
    return v;
  };
  auto cons_seg3 = [&](int c, int s) __attribute__((always_inline)) {
    if constexpr (!OUTW && !SAVE && !ROWS_NEXT) o_rows_out(c, s);
    const unsigned char* S = stage(s);
    const int olane = opaque_lane();
    const T* sK = reinterpret_cast<const T*>(S + L::sK);
    const T* sKn = reinterpret_cast<const T*>(S + L::sKn);
    const float* vec = reinterpret_cast<const float*>(S + L::sVec);
    const float eGC = vec[VEC_EGC * C];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const float f = vec[VEC_EGC_G * C + 16 * r + 4 * lg + s4];
#pragma unroll
        for (int j = 0; j < NTW; ++j) Z[r][j][s4] *= f;
      }
    if (eGC != 1.f) {  // (1 in every chunk of a lazy run that does not renormalise)
#pragma unroll
      for (int a = 0; a < KT; ++a)
#pragma unroll
        for (int j = 0; j < NTW; ++j) Ms[a][j] *= eGC;
    }
    const KnCols<DK> kcols(reinterpret_cast<const bf16*>(sKn), olane);  // bf16 only (unused for fp32)
#pragma unroll
    for (int kgi = 0; kgi < KGC; ++kgi) {
      frag bu[NTW];
#pragma unroll
      for (int j = 0; j < NTW; ++j) bu[j] = chain_frag<T>([&](int t) { return Z[t][j]; }, kgi);
#pragma unroll
      for (int a = 0; a < KT; ++a) {
        frag af;  // K^T rows 16a.., tokens of k-group kgi, from the row-major K tile
        if constexpr (MM::KG == 32) {
          const bf16* pa = kcols.tile(a) + 32 * kgi * DK;
          af = __builtin_shufflevector(tr_read(pa), tr_read(pa + 16 * DK), 0, 1, 2, 3, 4, 5, 6, 7);
        } else {
          af = lds_col4<T>(sK, LDK, 16 * kgi, 16 * a, lane);
        }
#pragma unroll
        for (int j = 0; j < NTW; ++j) MM::mma(Ms[a][j], af, bu[j]);
      }
    }
    if constexpr (OUTW) state_operands();  // the next chunk's state operands, for both waves
  };

  // Output wavefronts.  Segment 1: the state part of O^T, from the state
  // operands their consumer wave leaves in LDS.  Segment 2: P, masked with
  // the decay, four tiles per output wave (the producers form the other two),
  // into the fragment-order buffer.
  // Segment 3: U^T P^T and the store.
  auto outw_qm = [&](int s) __attribute__((always_inline)) {
#pragma unroll
    for (int kgi = 0; kgi < KGK; ++kgi) mfr[kgi][0] = sMx[kgi * 64 + lane];
    q_times_state(reinterpret_cast<const T*>(stage(s) + L::sQ), reinterpret_cast<const float*>(stage(s) + L::sVec));
  };
  auto outw_p = [&](auto wtag, int s) __attribute__((always_inline)) {
    using PT = OutPTiles<decltype(wtag)::value>;
    const unsigned char* S = stage(s);
    const T* sK = reinterpret_cast<const T*>(S + L::sK);
    const T* sQ = reinterpret_cast<const T*>(S + L::sQ);
    const float* vec = reinterpret_cast<const float*>(S + L::sVec);
    T* sPf = reinterpret_cast<T*>(smem + L::oPf);
    floatx4 pt[PT::n];  // lane holds P[16ti + lr][16tj + 4lg + s]
#pragma unroll
    for (int t = 0; t < PT::n; ++t) pt[t] = zero4();
    frag kf[KGK][4], qf[KGK][4];  // only the rows used are read, all before the first product
#pragma unroll
    for (int kgi = 0; kgi < KGK; ++kgi)
#pragma unroll
      for (int t = 0; t < PT::n; ++t) {
        kf[kgi][PT::tj[t]] = lds_frag(sK + (16 * PT::tj[t] + lr) * LDK, kgi, lane);
        qf[kgi][PT::ti[t]] = lds_frag(sQ + (16 * PT::ti[t] + lr) * LDK, kgi, lane);
      }
#pragma unroll
    for (int kgi = 0; kgi < KGK; ++kgi)
#pragma unroll
      for (int t = 0; t < PT::n; ++t) MM::mma(pt[t], kf[kgi][PT::tj[t]], qf[kgi][PT::ti[t]]);
#pragma unroll
    for (int t = 0; t < PT::n; ++t) {
      const floatx4 pv = pt[t] * decay_tile(vec, PT::ti[t], PT::tj[t], lg, lr);
      *reinterpret_cast<V4*>(sPf + L::pf(PT::ti[t], PT::tj[t], lane)) = pack4<T>(pv[0], pv[1], pv[2], pv[3]);
    }
  };

  // ------------------------------------------------------------ schedule
  // Producers and consumers run separate loops (so their registers are never
  // live at the same time) that execute the same sequence of barriers.  With
  // a double-buffered stage, iteration c runs three segments:
  //            producers                              consumers (chunk c)
  //   seg 1    inverses, P and -A of chunk c          Y = K M, Z, (Q M)^T; chunk c - 1's
  //                                                   output rows to HBM (ROWS_NEXT)
  //   seg 2    K, Q, V, gates of chunk c + 1;         U, O
  //            loads of chunk c + 2
  //   seg 3    Gram products of chunk c + 1           state update
  // With output wavefronts the consumers hand the state (after the update in
  // segment 3, for the next chunk) and U (segment 2) to them as bf16 operands,
  // and they form O^T: the state part in segment 1, P in segment 2 (all but
  // two tiles, which the producers form), U^T P^T and the store in segment 3.
  // Issue priority: consumers (the recurrence) over producers over output
  // waves; with output waves the producers' segment-1 work goes first.
  if (producer) {
    __builtin_amdgcn_s_setprio(1);
    if constexpr (MM::TPG == 2) {  // P tiles (0,1) and (2,3) share fragments with written tiles and are zero
      T* sPf = reinterpret_cast<T*>(smem + L::oPf);
      if (wave < 2) *reinterpret_cast<V4*>(sPf + L::pf(2 * wave, 2 * wave + 1, lane)) = pack4<T>(0.f, 0.f, 0.f, 0.f);
    }
    if (nch > 0) issue_loads(0);
    if constexpr (NSTAGE == 2) {
      if (nch > 0) {
        prod_stores(0, 0);
        lds_barrier();
        prod_gram(0);
        lds_barrier();
      }
      for (int c = 0; c < nch; ++c) {
        const bool more = c + 1 < nch;
        prod_finish(c & 1);
        lds_barrier();
        if (more) prod_stores(c + 1, (c + 1) & 1);
        lds_barrier();
        if (more) prod_gram((c + 1) & 1);
        lds_barrier();
      }
    } else {  // one stage: the two roles take turns
      for (int c = 0; c < nch; ++c) {
        prod_stores(c, 0);
        lds_barrier();
        prod_gram(0);
        lds_barrier();
        prod_finish(0);
        lds_barrier();
        lds_barrier();
        lds_barrier();
        lds_barrier();
      }
    }
  } else if (!consumer) {
    if constexpr (OUTW) {
      if (nch > 0) {
        lds_barrier();
        lds_barrier();
      }
      for (int c = 0; c < nch; ++c) {
        if constexpr (SAVE) {
          // a saving run writes no O: the output waves store the chunk's
          // starting state and U instead, from the consumers' operand copies
          save_state_from_operands(c);
          lds_barrier();
          lds_barrier();
          save_u_from_operands(c);
          lds_barrier();
        } else {
          outw_qm(c & 1);
          lds_barrier();
          if constexpr (NCW == 2) {
            if (wave == NP + NCW) outw_p(std::integral_constant<int, 0>(), c & 1);
            else outw_p(std::integral_constant<int, 1>(), c & 1);
          }
          lds_barrier();
          out_pu(c, c & 1, sUx);
          lds_barrier();
        }
      }
    }
  } else {
    __builtin_amdgcn_s_setprio(2);
    if constexpr (NSTAGE == 2) {
      if (nch > 0) {
        if constexpr (OUTW) state_operands();
        lds_barrier();
        lds_barrier();
      }
      for (int c = 0; c < nch; ++c) {
        if constexpr (SAVE && !OUTW) save_state(c);
        cons_seg1(c & 1);
        if constexpr (ROWS_NEXT) {
          if (c > 0) o_rows_out(c - 1, (c - 1) & 1);
        }
        lds_barrier();
        cons_seg2(c, c & 1);
        lds_barrier();
        cons_seg3(c, c & 1);
        lds_barrier();
      }
      if constexpr (ROWS_NEXT) {
        if (nch > 0) o_rows_out(nch - 1, (nch - 1) & 1);
      }
    } else {
      for (int c = 0; c < nch; ++c) {
        lds_barrier();
        lds_barrier();
        lds_barrier();
        if constexpr (SAVE && !OUTW) save_state(c);
        cons_seg1(0);
        lds_barrier();
        cons_seg2(c, 0);
        lds_barrier();
        cons_seg3(c, 0);
        lds_barrier();
      }
    }
  }

  if (consumer && nch > 0) {  // the state's scale after the last chunk
    const float lam = reinterpret_cast<const float*>(stage(NSTAGE == 2 ? (nch - 1) & 1 : 0) + L::sVec)[VEC_EGC * C + 1];
    if (lam != 1.f) {
#pragma unroll
      for (int a = 0; a < KT; ++a)
#pragma unroll
        for (int j = 0; j < NTW; ++j) Ms[a][j] *= lam;
    }
  }
  if constexpr (SEG) {  // every run's end state, for the scan over segments
    if (consumer) {
      float* e = (phi ? p.seg_phi : p.seg_fin) + ((static_cast<size_t>(seg) * p.batch + b) * p.Hv + h) * DK * DV;
#pragma unroll
      for (int a = 0; a < KT; ++a)
#pragma unroll
        for (int j = 0; j < NTW; ++j)
#pragma unroll
          for (int s = 0; s < 4; ++s) e[slane + MM::state_row(a, 0, s) * DV + 16 * j] = Ms[a][j][s];
    }
  } else if (consumer && p.hT) {
    float* hT = p.hT + sbase;
#pragma unroll
    for (int a = 0; a < KT; ++a)
#pragma unroll
      for (int j = 0; j < NTW; ++j)
#pragma unroll
        for (int s = 0; s < 4; ++s) hT[slane + MM::state_row(a, 0, s) * DV + 16 * j] = Ms[a][j][s];
  }
}

template <class T, int DK, int DV, int BV, int NSTAGE, int NCW, bool OUTW, bool SAVE, bool SEG = false>
hipError_t launch_cfg(const PrefillArgs& a, hipStream_t stream, const SegPlan* sp = nullptr) {
  using L = Layout<T, DK, BV, NSTAGE, NCW, OUTW>;
  static_assert(L::bytes <= 160 * 1024, "LDS budget of one gfx950 compute unit");
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
  p.save_state = a.save_state;
  p.save_u = a.save_u;
  p.chunk_base = a.chunk_base;
  p.order = a.order;
  p.T = a.seqlen;
  p.Hqk = a.Hqk;
  p.Hv = a.Hv;
  p.nslices = DV / BV;
  p.grp = a.Hv / a.Hqk;
  p.ngroups = a.num_seqs * a.Hqk;
  p.scale = a.scale;
  p.qt = nullptr;
  p.seg_fin = p.seg_phi = nullptr;
  p.seg_len = p.nseg = 0;
  p.batch = a.batch;
  if constexpr (SEG) {  // virtual sequences: every row's segments, later ones twice
    p.qt = sp->qt;
    p.seg_fin = sp->fin;
    p.seg_phi = sp->phi;
    p.seg_len = sp->seg_len;
    p.nseg = sp->nseg;
    p.grp = 2 * (a.Hv / a.Hqk);  // (segment 0 uses half of its group)
    p.ngroups = a.batch * sp->nseg * a.Hqk;
  }
  if (p.ngroups == 0) return hipSuccess;
  const int groups_pad = (p.ngroups + 7) / 8 * 8;
  const dim3 grid(groups_pad * p.grp * p.nslices);
  hipError_t e = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&prefill_kernel<T, DK, DV, BV, NSTAGE, NCW, OUTW, SAVE, SEG>),
      hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(L::bytes));
  if (e != hipSuccess) return e;
  prefill_kernel<T, DK, DV, BV, NSTAGE, NCW, OUTW, SAVE, SEG>
      <<<grid, dim3(64 * (NP + NCW * (OUTW ? 2 : 1))), L::bytes, stream>>>(p);
  return hipGetLastError();
}

template <class T, int DK, int DV, int BV, int NSTAGE, int NCW, bool OUTW>
hipError_t launch(const PrefillArgs& a, hipStream_t stream) {
  return a.save_state ? launch_cfg<T, DK, DV, BV, NSTAGE, NCW, OUTW, true>(a, stream)
                      : launch_cfg<T, DK, DV, BV, NSTAGE, NCW, OUTW, false>(a, stream);
}

// dv-slice width and consumer wavefronts.  Every (sequence, head) unit walks
// its chunks in order, so the time is the chunk count times the time per
// chunk of one workgroup.  With enough units to fill the 256 compute units,
// whole 128-column state rows per workgroup (four consumer wavefronts of two
// 16-column tiles each); with fewer, narrower slices: more workgroups, each
// redoing the chunk-local work but with fewer consumer wavefronts sharing its
// compute unit, which shortens the time per chunk.  (Narrower slices than 32
// columns do not shorten it further: with fewer units than compute units the
// time is still the chunk count times the same time per chunk.)
int slice_config(int units, int dv) {
  if (dv == 64) return units >= 128 ? 64 : 32;
  if (units >= 256) return 128;
  return units >= 128 ? 64 : 32;
}

// Longest-first order of packed sequences.  Each sequence's workgroups are
// numbered by its place in this order, so the dispatcher starts the longest
// sequences first and the short ones fill in at the end, instead of a long
// sequence that happens to come late setting the end of the launch (with
// lengths as uneven as a lognormal mix, that tail was a quarter of the time).
// Rank of sequence i = the number of sequences longer than it, or as long and
// before it: one thread per sequence, all lengths staged through LDS in turn.
constexpr int kMaxOrdered = kMaxOrderedSeqs;  // beyond this many sequences the natural order is kept

__global__ __launch_bounds__(256) void order_kernel(const int32_t* cu, int N, int32_t* order) {
  __shared__ int len[256];
  const int i = blockIdx.x * 256 + threadIdx.x;
  const int li = i < N ? cu[i + 1] - cu[i] : 0;
  int rank = 0;
  for (int j0 = 0; j0 < N; j0 += 256) {
    const int j = j0 + threadIdx.x;
    __syncthreads();
    len[threadIdx.x] = j < N ? cu[j + 1] - cu[j] : 0;
    __syncthreads();
    const int m = min(256, N - j0);
    for (int u = 0; u < m; ++u) {
      const int lj = len[u];
      rank += (lj > li) | ((lj == li) & (j0 + u < i));
    }
  }
  if (i < N) order[rank] = i;
}
}  // namespace

// Scratch of the allocation-free prefill (launch_prefill_noalloc): the longest-first order of up to
// kMaxOrdered packed sequences, 16 KiB.  Every GPU the library runs on holds its own copy until the
// process ends.  In host code the name stands for a host-side handle, not a device address: host code
// uses only the per-device address hipGetSymbolAddress returns (noalloc_scratch below).
static __device__ __align__(256) int32_t scratch[kMaxOrdered];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<int32_t*> g_scratch[kMaxDevices];  // the address of scratch on each device, looked up once

// The current device's copy of scratch.  Two threads that both find it missing look up the same
// address and store the same value.
hipError_t noalloc_scratch(int32_t** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  int32_t* ptr = g_scratch[dev].load(std::memory_order_acquire);
  if (!ptr) {
    void* sym = nullptr;
    e = hipGetSymbolAddress(&sym, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    ptr = static_cast<int32_t*>(sym);
    g_scratch[dev].store(ptr, std::memory_order_release);
  }
  *out = ptr;
  return hipSuccess;
}

// The fused kernel in the configuration the unit count selects (no workspace).
hipError_t launch_fused(const PrefillArgs& a, hipStream_t stream) {
  const int units = a.num_seqs * a.Hv;
  if (a.bf16) {
    if (a.dk == 128 && a.dv == 128) {
      switch (slice_config(units, 128)) {
        case 128: return launch<bf16, 128, 128, 128, 2, 4, false>(a, stream);
        case 64: return launch<bf16, 128, 128, 64, 2, 4, false>(a, stream);
        default: return launch<bf16, 128, 128, 32, 2, 2, true>(a, stream);
      }
    }
    if (a.dk == 64 && a.dv == 64)
      return slice_config(units, 64) == 64 ? launch<bf16, 64, 64, 64, 2, 4, false>(a, stream)
                                           : launch<bf16, 64, 64, 32, 2, 2, true>(a, stream);
  } else {
    if (a.dk == 64 && a.dv == 64) return launch<float, 64, 64, 64, 1, 4, false>(a, stream);
  }
  return hipErrorInvalidValue;
}
}  // namespace


hipError_t launch_prefill(const PrefillArgs& args, hipStream_t stream) {
  if (args.chunk != C) return hipErrorInvalidValue;
  PrefillArgs a = args;
  if (a.cu_seqlens && !a.save_state && a.workspace && order_workspace_bytes(a.num_seqs) &&
      a.workspace_bytes >= order_workspace_bytes(a.num_seqs)) {
    int32_t* order = static_cast<int32_t*>(a.workspace);
    order_kernel<<<dim3((a.num_seqs + 255) / 256), dim3(256), 0, stream>>>(a.cu_seqlens, a.num_seqs, order);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    a.order = order;
  }
  // A few long rows: segments side by side, finished by a scan and a correction.
  if (a.bf16 && a.dk == 128 && a.dv == 128 && !a.cu_seqlens && !a.save_state && a.workspace) {
    SegPlan sp;
    if (seg_plan(a.batch, a.seqlen, a.Hv, &sp) &&
        a.workspace_bytes >= seg_workspace_bytes(a.batch, a.seqlen, a.Hv)) {
      seg_carve(a.workspace, a.batch, a.seqlen, a.Hv, &sp);
      const hipError_t e = launch_cfg<bf16, 128, 128, 128, 2, 4, false, false, true>(a, stream, &sp);
      if (e != hipSuccess) return e;
      return launch_seg_finish(a, sp, stream);
    }
  }
  return launch_fused(a, stream);
}

hipError_t launch_prefill_noalloc(const PrefillArgs& args, hipStream_t stream) {
  if (args.chunk != C || args.save_state || args.num_seqs > kMaxOrdered) return hipErrorInvalidValue;
  PrefillArgs a = args;
  a.workspace = nullptr;
  a.workspace_bytes = 0;
  if (a.cu_seqlens && order_workspace_bytes(a.num_seqs)) {
    int32_t* order = nullptr;
    hipError_t e = noalloc_scratch(&order);
    if (e != hipSuccess) return e;
    order_kernel<<<dim3((a.num_seqs + 255) / 256), dim3(256), 0, stream>>>(a.cu_seqlens, a.num_seqs, order);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    a.order = order;
  }
  return launch_fused(a, stream);
}

}  // namespace gdn

// LDS layouts, operand reads and staging shared by the chunked prefill kernels
// (the fused kernel in prefill.hip and the two-pass scan in scan.hip): the
// chunk length, the swizzles of the V tile and of the column-read copy of K,
// the per-token gate vectors and decay factors, and the producers' loads and
// stores of one chunk.
#pragma once

#include "device_common.hpp"

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
  __device__ __forceinline__ void load_kqv(const T* kb, const T* qb, const T* vb, uint32_t qk_row, uint32_t v_row,
                                           int Lc, int tid, bool vzero = false) {
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
  }
  // K, Q and V as above, and the gates (g, beta) of the chunk's tokens on the last producer wave.
  __device__ __forceinline__ void load(const T* kb, const T* qb, const T* vb, uint32_t qk_row, uint32_t v_row,
                                       const float* gb, const float* bb, uint32_t g_row, int Lc, int tid,
                                       bool vzero = false) {
    load_kqv(kb, qb, vb, qk_row, v_row, Lc, tid, vzero);
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

}  // namespace
}  // namespace gdn

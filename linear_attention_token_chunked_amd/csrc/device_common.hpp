// Device-side helpers shared by the gfx950 kernels: element types, conversions
// and the two matrix-core primitives the prefill kernels are written against.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace gdn {

typedef __bf16 bf16;
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef unsigned uintx2 __attribute__((ext_vector_type(2)));
typedef unsigned uintx4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float to_float(float x) { return x; }
__device__ __forceinline__ float to_float(bf16 x) { return static_cast<float>(x); }

template <class T>
__device__ __forceinline__ T from_float(float x);
template <>
__device__ __forceinline__ float from_float<float>(float x) { return x; }
template <>
__device__ __forceinline__ bf16 from_float<bf16>(float x) { return static_cast<bf16>(x); }  // RNE

// Four consecutive elements of type T as one vector store/load unit.
template <class T> struct Vec4;
template <> struct Vec4<float> { typedef floatx4 type; };
template <> struct Vec4<bf16> { typedef bf16x4 type; };

// Two floats rounded to nearest even bf16, a in the low half.  Written as one
// two-element conversion: element-wise casts into a 4- or 8-element bf16 vector
// are emitted as one conversion per value plus byte permutes, three times the
// instructions (and on a dependent chain, three times the latency).
__device__ __forceinline__ unsigned pk_bf16(float a, float b) {
  return __builtin_bit_cast(unsigned, __builtin_convertvector(floatx2{a, b}, bf16x2));
}

template <class T>
__device__ __forceinline__ typename Vec4<T>::type pack4(float a, float b, float c, float d) {
  if constexpr (sizeof(T) == 2) {
    return __builtin_bit_cast(bf16x4, uintx2{pk_bf16(a, b), pk_bf16(c, d)});
  } else {
    return floatx4{a, b, c, d};
  }
}

// pack4 of (-a, -b, -c, -d): for bf16 the sign bits are flipped after the
// rounding (exact, since rounding to nearest even is symmetric), one xor per
// pair instead of one per value.
template <class T>
__device__ __forceinline__ typename Vec4<T>::type pack4_neg(float a, float b, float c, float d) {
  if constexpr (sizeof(T) == 2) {
    return __builtin_bit_cast(bf16x4, uintx2{pk_bf16(a, b) ^ 0x80008000u, pk_bf16(c, d) ^ 0x80008000u});
  } else {
    return floatx4{-a, -b, -c, -d};
  }
}

// ---------------------------------------------------------------------------
// Matrix-core fragments.
//
// Every product in the prefill kernels is built from 16x16 output tiles on one
// 64-lane wavefront.  The accumulator ("D layout") of a 16x16 tile gives lane l
// the four elements D[4*(l/16) + s][l%16], s = 0..3.
//
// A "k-group" is the slice of the contraction dimension one fragment covers:
// 32 values for bf16 (one v_mfma_f32_16x16x32_bf16) and 16 values for fp32 (four
// v_mfma_f32_16x16x4_f32).  Either way a lane holds 16 bytes of A and 16 bytes
// of B per k-group: A[l%16][k in K(l/16)] and B[k in K(l/16)][l%16], with the
// same k set K(g) on both sides, so the sum runs over the whole k-group whatever
// the order inside it.
//
// The order is chosen so that accumulator tiles can be fed back into the next
// product straight from registers ("chaining"): lane group g owns accumulator
// rows 4g..4g+3, so K(g) is taken to be {4g..4g+3} for fp32 and
// {4g..4g+3} u {16+4g..16+4g+3} for bf16 (two stacked accumulator tiles).
// Operands read from LDS rows instead come in natural k order: lane group g
// reads k = 8g..8g+7 of a bf16 k-group as one 16-byte run.  Where both meet (the
// state, a chained B operand, against K or Q rows from LDS), the state's
// accumulator rows are assigned to key indices to match (see state_row).
template <class T> struct Mma;

template <> struct Mma<bf16> {
  typedef bf16x8 frag;
  static constexpr int KG = 32;   // contraction values per k-group
  static constexpr int TPG = 2;   // accumulator tiles per k-group when chaining
  __device__ __forceinline__ static void mma(floatx4& c, const frag& a, const frag& b) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  // Operand fragment from the two accumulator tiles that cover one k-group.
  __device__ __forceinline__ static frag chain(const floatx4& lo, const floatx4& hi) {
    return __builtin_bit_cast(frag, uintx4{pk_bf16(lo[0], lo[1]), pk_bf16(lo[2], lo[3]), pk_bf16(hi[0], hi[1]),
                                           pk_bf16(hi[2], hi[3])});
  }
  // Key index held by row 4g + s of state accumulator tile a.  Element e of
  // the chained operand of k-group kg is row 4g + (e & 3) of tile 2kg + (e >> 2);
  // it must pair with key 32kg + 8g + e, the one a natural-order LDS row
  // gives lane group g there.
  __device__ __forceinline__ static constexpr int state_row(int a, int g, int s) {
    return 32 * (a >> 1) + 8 * g + 4 * (a & 1) + s;
  }
};

template <> struct Mma<float> {
  typedef floatx4 frag;
  static constexpr int KG = 16;
  static constexpr int TPG = 1;
  __device__ __forceinline__ static void mma(floatx4& c, const frag& a, const frag& b) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], c, 0, 0, 0);
  }
  __device__ __forceinline__ static frag chain(const floatx4& t) { return t; }
  __device__ __forceinline__ static constexpr int state_row(int a, int g, int s) { return 16 * a + 4 * g + s; }
};

// 16-byte operand fragment of k-group kg from an LDS row (row-major, natural
// k order).  Lane group g reads bytes [16g, 16g+16) of the group.
template <class T>
__device__ __forceinline__ typename Mma<T>::frag lds_frag(const T* row, int kg, int lane) {
  constexpr int EPB = 16 / sizeof(T);
  return *reinterpret_cast<const typename Mma<T>::frag*>(row + kg * Mma<T>::KG + (lane >> 4) * EPB);
}

__device__ __forceinline__ floatx4 zero4() { return floatx4{0.f, 0.f, 0.f, 0.f}; }

constexpr float kLog2e = 1.4426950408889634f;

// Floor of a log-gate g = log(alpha) before it enters an in-chunk prefix sum.
// alpha = 0 (a full forget) arrives as g = -inf, and differences of prefix sums
// would then be -inf - (-inf) = NaN.  exp(-200) is below the smallest fp32
// value, so every decay factor that spans a floored token is still exactly 0,
// as for alpha = 0, while the sums stay finite (a few floored tokens in a chunk
// keep them within a few thousand, where fp32 resolves differences to 1e-3 or
// better).  Gates at or above the floor are unchanged.
constexpr float kGateFloor = -200.f;

// Inclusive prefix sum over the 64 lanes of a wavefront with DPP row shifts
// and row broadcasts (no LDS round trips).
__device__ __forceinline__ float wave_inclusive_sum(float x) {
#define GDN_DPP_ADD(ctrl, rows)                                                                               \
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), ctrl, rows, 0xf, false))
  GDN_DPP_ADD(0x111, 0xf);  // row_shr:1
  GDN_DPP_ADD(0x112, 0xf);  // row_shr:2
  GDN_DPP_ADD(0x114, 0xf);  // row_shr:4
  GDN_DPP_ADD(0x118, 0xf);  // row_shr:8
  GDN_DPP_ADD(0x142, 0xa);  // row_bcast:15 into rows 1 and 3
  GDN_DPP_ADD(0x143, 0xc);  // row_bcast:31 into rows 2 and 3
#undef GDN_DPP_ADD
  return x;
}

// Every lane gets x from lane S of its group of four (DPP quad permutation).
template <int S>
__device__ __forceinline__ float quad_bcast(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x55 * S, 0xf, 0xf, false));
}

// Column cc of (I + A)^-1 for a 16x16 strictly lower A by right-looking
// forward substitution, four lanes per column: the lane with q = lane % 4
// holds rows 4q..4q+3 in x.  Once x_j is final (step j) it is broadcast
// within the quad and every row i > j takes x_i -= A_ij x_j; At[j][i] = A_ij
// (zero for i <= j, so the other rows are unchanged).
// The 15 columns of A the lane needs are loaded first, so the substitution
// waits for LDS once rather than once per step.
template <int... J>
__device__ __forceinline__ void unit_lower_inverse_column(floatx4& x, const float* At, int ld, int q,
                                                          std::integer_sequence<int, J...>) {
  floatx4 a[sizeof...(J)];
  ((a[J] = *reinterpret_cast<const floatx4*>(At + J * ld + 4 * q)), ...);
  ((x -= a[J] * quad_bcast<J / 4>(x[J % 4])), ...);
}

// 16x16 tile products whose contraction is one 16-wide block: lane group g
// supplies k = 4g..4g+3, which is the row set it owns in an accumulator tile.
template <class T> struct Mma16;
template <> struct Mma16<bf16> {
  typedef bf16x4 frag;
  __device__ __forceinline__ static void mma(floatx4& c, const frag& a, const frag& b) {
    typedef short s4 __attribute__((ext_vector_type(4)));
    c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s4, a), __builtin_bit_cast(s4, b), c, 0, 0,
                                                   0);
  }
  __device__ __forceinline__ static frag chain(const floatx4& t) {
    return __builtin_bit_cast(frag, uintx2{pk_bf16(t[0], t[1]), pk_bf16(t[2], t[3])});
  }
};
template <> struct Mma16<float> {
  typedef floatx4 frag;
  __device__ __forceinline__ static void mma(floatx4& c, const frag& a, const frag& b) { Mma<float>::mma(c, a, b); }
  __device__ __forceinline__ static frag chain(const floatx4& t) { return t; }
};

// Four consecutive rows of one column of a row-major LDS tile, as lane data
// for the accumulator layout: lane (lg, lr) gets X[r0 + 4lg + e][c0 + lr],
// e = 0..3 (c0 a multiple of 16).  bf16 uses the gfx950 transposing LDS read:
// in each 16-lane group, lane i returns element i%4 of the 8-byte loads of
// lanes 4e + i/4, so lane j loads row r0 + 4lg + j/4 at the 4-column run
// c0 + 4(j%4).  fp32 reads the four values one by one.
template <class T>
__device__ __forceinline__ typename Vec4<T>::type lds_col4(const T* base, int ld, int r0, int c0, int lane) {
  const int lg = lane >> 4, lr = lane & 15;
  if constexpr (sizeof(T) == 2) {
    typedef short s4 __attribute__((ext_vector_type(4)));
    const T* ptr = base + (r0 + 4 * lg + (lr >> 2)) * ld + c0 + 4 * (lr & 3);
    const s4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        reinterpret_cast<__attribute__((address_space(3))) s4*>(reinterpret_cast<size_t>(ptr)));
    return __builtin_bit_cast(typename Vec4<T>::type, v);
  } else {
    typename Vec4<T>::type v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = base[(r0 + 4 * lg + e) * ld + c0 + lr];
    return v;
  }
}

// Workgroup barrier that orders LDS only: waits for this wave's LDS (and
// scalar) operations, then s_barrier.  Unlike __syncthreads() it does not wait
// for outstanding global loads, so loads issued ahead of time (the next
// chunk's operands) stay in flight across it.  The "memory" clobber keeps the
// compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

}  // namespace gdn

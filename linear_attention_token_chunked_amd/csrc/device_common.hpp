// Device-side helpers shared by the gfx950 kernels: element types, conversions
// and the two matrix-core primitives the prefill kernels are written against.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16;
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
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

template <class T>
__device__ __forceinline__ typename Vec4<T>::type pack4(float a, float b, float c, float d) {
  typename Vec4<T>::type r;
  r[0] = from_float<T>(a);
  r[1] = from_float<T>(b);
  r[2] = from_float<T>(c);
  r[3] = from_float<T>(d);
  return r;
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
    frag f;
    f[0] = static_cast<bf16>(lo[0]); f[1] = static_cast<bf16>(lo[1]);
    f[2] = static_cast<bf16>(lo[2]); f[3] = static_cast<bf16>(lo[3]);
    f[4] = static_cast<bf16>(hi[0]); f[5] = static_cast<bf16>(hi[1]);
    f[6] = static_cast<bf16>(hi[2]); f[7] = static_cast<bf16>(hi[3]);
    return f;
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

// Workgroup barrier that orders LDS only: waits for this wave's LDS (and
// scalar) operations, then s_barrier.  Unlike __syncthreads() it does not wait
// for outstanding global loads, so loads issued ahead of time (the next
// chunk's operands) stay in flight across it.  The "memory" clobber keeps the
// compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

}  // namespace gdn

// Cross-lane sums and the state write shared by the single decode step and
// the multi-token verify (decode.hip, verify.hip), gfx950.  Both kernels take
// every sum and every write through these, so that a verify over Tv tokens
// equals Tv single steps bit for bit.
#pragma once

#include "device_common.hpp"

namespace gdn {

// Cross-lane sums of the single step and the multi-token verify, which share them so that a verify
// equals repeated single steps bit for bit.  add_xor9<OFF> adds to each of nine values its copy in lane
// l ^ OFF (both lanes of a pair get the same bits): a DPP rotation of the 16-lane rows by 8 for OFF = 8,
// the gfx950 row swaps for OFF = 16 and 32, a lane shuffle otherwise.  A row swap exchanges whole rows
// between its two registers, so two copies of x end as the two halves of every pair (v_permlane16_swap:
// the odd rows of the first with the even rows of the second; v_permlane32_swap: the upper half of the
// first with the lower half of the second).  They are written out because this compiler returns the
// first register for both results of the builtins.  No operand is a memory access.
#define GDN_SWAP9(op)                                                                                          \
  asm volatile("s_nop 1\n\t" op " %0, %9\n\t" op " %1, %10\n\t" op " %2, %11\n\t" op " %3, %12\n\t" op " %4, %13\n\t" op \
               " %5, %14\n\t" op " %6, %15\n\t" op " %7, %16\n\t" op " %8, %17\n\ts_nop 1"                            \
               : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(a[4]), "+v"(a[5]), "+v"(a[6]), "+v"(a[7]),     \
                 "+v"(a[8]), "+v"(b[0]), "+v"(b[1]), "+v"(b[2]), "+v"(b[3]), "+v"(b[4]), "+v"(b[5]), "+v"(b[6]),     \
                 "+v"(b[7]), "+v"(b[8]))
template <int OFF>
__device__ __forceinline__ void add_xor9(float (&x)[9]) {
  if constexpr (OFF == 8) {
#pragma unroll
    for (int i = 0; i < 9; ++i)
      x[i] += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x[i]), 0x128, 0xf, 0xf,
                                                                    false));  // row_ror:8
  } else if constexpr (OFF == 16 || OFF == 32) {
    float a[9], b[9];
#pragma unroll
    for (int i = 0; i < 9; ++i) a[i] = b[i] = x[i];
    if constexpr (OFF == 16)
      GDN_SWAP9("v_permlane16_swap_b32");
    else
      GDN_SWAP9("v_permlane32_swap_b32");
#pragma unroll
    for (int i = 0; i < 9; ++i) x[i] = a[i] + b[i];
  } else {
#pragma unroll
    for (int i = 0; i < 9; ++i) x[i] += __shfl_xor(x[i], OFF);
  }
}
#undef GDN_SWAP9
// Sum of each value over the lanes l ^ j, j a multiple of OFF (a power of two below 64): a butterfly
// from OFF up.
template <int OFF>
__device__ __forceinline__ void xor_sums9(float (&x)[9]) {
  if constexpr (OFF < 64) {
    add_xor9<OFF>(x);
    xor_sums9<2 * OFF>(x);
  }
}
// One recurrent write to four state columns, alpha m + k u, in the rounding order both kernels share:
// alpha m rounded, then k u added by one fused multiply-add (which updates the state registers in place).
__device__ __forceinline__ floatx4 decay_write(const floatx4& m, float alpha, float k, const floatx4& u) {
  floatx4 r;
#pragma unroll
  for (int c = 0; c < 4; ++c) r[c] = __builtin_fmaf(k, u[c], alpha * m[c]);
  return r;
}

}  // namespace gdn

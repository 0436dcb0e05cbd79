// Output epilogue of the GDN layer: zero-centred RMSNorm and a sigmoid output
// gate over every (token, value head) row of the mixer output, gfx950.
//
// The podcast transcript on "On the Design of Qwen3.8-Next Architecture"
// (cue 14) lists what the model adds around the gated delta rule: a sigmoid
// output gate and a zero-centred RMSNorm; the archdiff model page
// "Qwen3.8-2.4T-A95B" (components list) writes the gate as sigmoid(x W_g)
// times o.  Per row o of dv values, with gate pre-activations z and a
// zero-centred weight w (the scale is 1 + w):
//   y = sigmoid(z) * (o / sqrt(mean(o^2) + eps)) * (1 + w).
// The kernel is bound by HBM bandwidth: it reads o and z once and writes y
// once.  Sixteen lanes share a row (for 128 values: 16 bytes of bf16, or 32
// of fp32, per lane), so a wavefront covers four rows and the row sums reduce
// inside 16-lane groups.
#include "device_common.hpp"
#include "launch.hpp"

namespace gdn {
namespace {

constexpr int kEpiThreads = 256;
// Rows per 16-lane group: a workgroup covers 16 kEpiRows consecutive rows, group g rows g, g + 16, ...
// All of a lane's loads are issued before the first row is formed.  Loads and stores stream
// (non-temporal): every byte is touched once, and the output is read again only by the next layer,
// after much else (on a 5 GB output the streaming loads took the call from 907 to 847 us).  Each lane
// writes exactly the elements it read, so y may be o.
constexpr int kEpiRows = 4;

// Sum over the 16 lanes of a DPP row (lanes 16r .. 16r + 15), the same bits in every lane, without
// LDS: lanes i and 7 - i of each half-row (half-row mirror), then pairs l ^ 1 and l ^ 2 (quad
// permutations), then l ^ 8 (rotation of the row by 8).
template <int CTRL>
__device__ __forceinline__ float dpp_plus(float x) {
  return x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float row16_sum(float x) {
  x = dpp_plus<0x141>(x);  // row_half_mirror
  x = dpp_plus<0xb1>(x);   // quad_perm [1, 0, 3, 2]
  x = dpp_plus<0x4e>(x);   // quad_perm [2, 3, 0, 1]
  return dpp_plus<0x128>(x);  // row_ror:8
}

template <class T, int DV>
__global__ __launch_bounds__(kEpiThreads) void norm_gate_kernel(const T* o, const T* __restrict__ z,
                                                                const float* __restrict__ w, T* y, int64_t rows,
                                                                float eps) {
  constexpr int EPL = DV / 16;  // values per lane (16 lanes per row)
  constexpr int R = kEpiRows;
  static_assert(EPL == 4 || EPL == 8, "dv of 64 or 128");
  const int lane16 = threadIdx.x & 15;
  typedef T lane_vec __attribute__((ext_vector_type(EPL)));
  typedef float lane_wvec __attribute__((ext_vector_type(EPL)));
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * (kEpiThreads / 16) * R + (threadIdx.x >> 4);
  const lane_wvec w_in = *reinterpret_cast<const lane_wvec*>(w + lane16 * EPL);
  lane_vec o_in[R], z_in[R];
#pragma unroll
  for (int i = 0; i < R; ++i) {  // (rows past the end read the last row: never stored)
    const int64_t row = min(row0 + i * (kEpiThreads / 16), rows - 1);
    o_in[i] = __builtin_nontemporal_load(reinterpret_cast<const lane_vec*>(o + row * DV + lane16 * EPL));
    z_in[i] = __builtin_nontemporal_load(reinterpret_cast<const lane_vec*>(z + row * DV + lane16 * EPL));
  }
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int64_t row = row0 + i * (kEpiThreads / 16);
    float ov[EPL], zv[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      ov[e] = to_float(o_in[i][e]);
      zv[e] = to_float(z_in[i][e]);
    }
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) ss += ov[e] * ov[e];
    ss = row16_sum(ss);
    const float rinv = rsqrtf(ss * (1.f / DV) + eps);
    float out[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      // sigmoid(z) = 1 / (1 + 2^(-z log2 e)) with the hardware base-2 exponential and reciprocal,
      // each within about an ulp of fp32 (for very negative z, 2^x overflows to inf: the gate is 0)
      const float gate = __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-zv[e] * kLog2e));
      out[e] = gate * (ov[e] * rinv) * (1.f + w_in[e]);
    }
    if (row < rows) {
      lane_vec yv;
#pragma unroll
      for (int e = 0; e < EPL; ++e) yv[e] = from_float<T>(out[e]);
      __builtin_nontemporal_store(yv, reinterpret_cast<lane_vec*>(y + row * DV + lane16 * EPL));
    }
  }
}

template <class T, int DV>
hipError_t launch(const EpilogueArgs& a, hipStream_t stream) {
  if (a.rows == 0) return hipSuccess;
  const int64_t per_wg = kEpiThreads / 16 * kEpiRows;
  const dim3 grid(static_cast<unsigned>((a.rows + per_wg - 1) / per_wg));
  norm_gate_kernel<T, DV><<<grid, dim3(kEpiThreads), 0, stream>>>(
      static_cast<const T*>(a.o), static_cast<const T*>(a.z), a.weight, static_cast<T*>(a.y), a.rows, a.eps);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_norm_gate(const EpilogueArgs& a, hipStream_t stream) {
  if (a.dv == 128) return a.bf16 ? launch<bf16, 128>(a, stream) : launch<float, 128>(a, stream);
  if (a.dv == 64) return a.bf16 ? launch<bf16, 64>(a, stream) : launch<float, 64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace gdn

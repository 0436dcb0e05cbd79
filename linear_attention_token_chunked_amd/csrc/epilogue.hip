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

// Sum over the 16 lanes of a DPP row (lanes 16r .. 16r + 15).
__device__ __forceinline__ float row16_sum(float x) {
  x += __shfl_xor(x, 1);
  x += __shfl_xor(x, 2);
  x += __shfl_xor(x, 4);
  x += __shfl_xor(x, 8);
  return x;
}

template <class T, int DV>
__global__ __launch_bounds__(kEpiThreads) void norm_gate_kernel(const T* o, const T* __restrict__ z,
                                                                const float* __restrict__ w, T* y, int64_t rows,
                                                                float eps) {
  constexpr int EPL = DV / 16;  // values per lane (16 lanes per row)
  static_assert(EPL == 4 || EPL == 8, "dv of 64 or 128");
  const int lane16 = threadIdx.x & 15;
  const int64_t row = (static_cast<int64_t>(blockIdx.x) * kEpiThreads + threadIdx.x) >> 4;
  if (row >= rows) return;  // whole 16-lane groups leave together
  typedef T lane_vec __attribute__((ext_vector_type(EPL)));  // a lane's run: one or two 16-byte pieces
  typedef float lane_wvec __attribute__((ext_vector_type(EPL)));
  const int64_t base = row * DV + lane16 * EPL;
  const lane_vec o_in = *reinterpret_cast<const lane_vec*>(o + base);
  const lane_vec z_in = *reinterpret_cast<const lane_vec*>(z + base);
  const lane_wvec w_in = *reinterpret_cast<const lane_wvec*>(w + lane16 * EPL);
  float ov[EPL], zv[EPL], wv[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    ov[e] = to_float(o_in[e]);
    zv[e] = to_float(z_in[e]);
    wv[e] = w_in[e];
  }
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < EPL; ++e) ss += ov[e] * ov[e];
  ss = row16_sum(ss);
  const float rinv = rsqrtf(ss * (1.f / DV) + eps);
  float out[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    const float gate = 1.f / (1.f + expf(-zv[e]));
    out[e] = gate * (ov[e] * rinv) * (1.f + wv[e]);
  }
#pragma unroll
  for (int e = 0; e < EPL; e += 4)
    *reinterpret_cast<typename Vec4<T>::type*>(y + base + e) = pack4<T>(out[e], out[e + 1], out[e + 2], out[e + 3]);
}

template <class T, int DV>
hipError_t launch(const EpilogueArgs& a, hipStream_t stream) {
  if (a.rows == 0) return hipSuccess;
  const int64_t threads = a.rows * 16;
  const dim3 grid(static_cast<unsigned>((threads + kEpiThreads - 1) / kEpiThreads));
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

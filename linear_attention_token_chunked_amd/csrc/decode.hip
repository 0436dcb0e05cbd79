// Single-token decode step of the gated delta rule (one workgroup per
// (sequence, value head)), gfx950.
//
// The step is the recurrence from the podcast transcript on "On the Design of
// Qwen3.8-Next Architecture" (cue 14: decay the state, read under the key,
// write the error), applied in the stored layout M = S^T (dk x dv):
//   r = M^T k, p = M^T q            (one read pass over M)
//   u = beta (v - alpha r)
//   o = scale (alpha p + (k.q) u)   (= M_new^T q)
//   M <- alpha M + k u^T            (one write pass)
// Each state element is read once and written once, so the kernel is bound by
// HBM bandwidth: a workgroup streams its dk x dv fp32 slice (64 KiB at 128x128)
// with 16-byte loads, keeps it in registers across the dk-reduction, and
// writes it back.
#include "device_common.hpp"
#include "lane_sums.hpp"
#include "launch.hpp"

namespace gdn {
namespace {

constexpr int kDecodeThreads = 256;

template <class T, int DK, int DV>
__global__ __launch_bounds__(kDecodeThreads) void decode_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, float* __restrict__ state,
    T* __restrict__ o, int Hqk, int Hv, float scale) {
  // Each wavefront owns a block of DV / 4 state columns over all DK rows, so the
  // reductions over the key dimension stay inside the wavefront (DPP and row
  // swaps, no LDS).  A thread holds rows rg, rg + RG, ... of four columns, so a load
  // instruction covers RG consecutive rows.
  constexpr int NWAVE = kDecodeThreads / 64;
  constexpr int CPW = DV / NWAVE;  // state columns per wavefront
  constexpr int TPR = CPW / 4;     // threads per row of them (one float4 each)
  constexpr int RG = 64 / TPR;     // row groups of a wavefront
  constexpr int RPT = DK / RG;     // rows per thread: rg, rg + RG, ...
  static_assert(CPW % 4 == 0 && 64 % TPR == 0 && DK % RG == 0, "shape");

  const int unit = blockIdx.x;  // n * Hv + h
  const int n = unit / Hv;
  const int h = unit - n * Hv;
  const int hq = h / (Hv / Hqk);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int rg = lane / TPR;
  const int col = (tid >> 6) * CPW + 4 * (lane % TPR);

  __shared__ float sk[DK];
  __shared__ float sq[DK];

  // Issue the whole state slice first: these loads dominate the run time.
  float* M = state + static_cast<size_t>(unit) * DK * DV;
  floatx4 m[RPT];
#pragma unroll
  for (int r = 0; r < RPT; ++r)
    m[r] = *reinterpret_cast<const floatx4*>(M + static_cast<size_t>(rg + RG * r) * DV + col);

  const T* kp = k + (static_cast<size_t>(n) * Hqk + hq) * DK;
  const T* qp = q + (static_cast<size_t>(n) * Hqk + hq) * DK;
  for (int i = tid; i < DK; i += kDecodeThreads) {
    sk[i] = to_float(kp[i]);
    sq[i] = to_float(qp[i]);
  }
  const float alpha = expf(g[unit]);
  const float b = beta[unit];
  const T* vp = v + static_cast<size_t>(unit) * DV + col;
  const float v0 = to_float(vp[0]), v1 = to_float(vp[1]), v2 = to_float(vp[2]), v3 = to_float(vp[3]);
  __syncthreads();

  floatx4 r = zero4(), p = zero4();
  float kq = 0.f;
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const float ki = sk[rg + RG * i], qi = sq[rg + RG * i];
    r += ki * m[i];
    p += qi * m[i];
    kq += ki * qi;
  }
  // Sum over the wavefront's row groups: every lane ends with the full sums of its columns.
  {
    float x9[9] = {r[0], r[1], r[2], r[3], p[0], p[1], p[2], p[3], kq};
    xor_sums9<TPR>(x9);
    r = floatx4{x9[0], x9[1], x9[2], x9[3]};
    p = floatx4{x9[4], x9[5], x9[6], x9[7]};
    kq = x9[8];
  }
  floatx4 u;
  u[0] = b * (v0 - alpha * r[0]);
  u[1] = b * (v1 - alpha * r[1]);
  u[2] = b * (v2 - alpha * r[2]);
  u[3] = b * (v3 - alpha * r[3]);

  // The updated state is not read again until the next step, after the rest of
  // the state (and, in a model, every other layer) has streamed through the
  // caches, so it is written with non-temporal stores.  Measured on MI355X at
  // 256 sequences x 32 heads: 6.4 TB/s against 5.1 TB/s with ordinary stores
  // (non-temporal loads, by contrast, are slower).
#pragma unroll
  for (int i = 0; i < RPT; ++i)
    __builtin_nontemporal_store(decay_write(m[i], alpha, sk[rg + RG * i], u),
                                reinterpret_cast<floatx4*>(M + static_cast<size_t>(rg + RG * i) * DV + col));
  if (rg == 0) {
    const floatx4 ov = scale * (alpha * p + kq * u);
    *reinterpret_cast<typename Vec4<T>::type*>(o + static_cast<size_t>(unit) * DV + col) =
        pack4<T>(ov[0], ov[1], ov[2], ov[3]);
  }
}

template <class T, int DK, int DV>
hipError_t launch(const DecodeArgs& a, hipStream_t stream) {
  const int units = a.num_seqs * a.Hv;
  if (units == 0) return hipSuccess;
  decode_kernel<T, DK, DV><<<dim3(units), dim3(kDecodeThreads), 0, stream>>>(
      static_cast<const T*>(a.q), static_cast<const T*>(a.k), static_cast<const T*>(a.v), a.g, a.beta,
      a.state, static_cast<T*>(a.o), a.Hqk, a.Hv, a.scale);
  return hipGetLastError();
}

template <class T>
hipError_t dispatch_dims(const DecodeArgs& a, hipStream_t stream) {
  if (a.dk == 128 && a.dv == 128) return launch<T, 128, 128>(a, stream);
  if (a.dk == 64 && a.dv == 64) return launch<T, 64, 64>(a, stream);
  if (a.dk == 128 && a.dv == 64) return launch<T, 128, 64>(a, stream);
  if (a.dk == 64 && a.dv == 128) return launch<T, 64, 128>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  return a.bf16 ? dispatch_dims<bf16>(a, stream) : dispatch_dims<float>(a, stream);
}

}  // namespace gdn

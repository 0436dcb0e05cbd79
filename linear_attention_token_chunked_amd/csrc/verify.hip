// Multi-token verify from a live state: Tv consecutive recurrent steps per
// (sequence, value head) in one pass over the state, gfx950.
//
// Speculative decoding drafts a few tokens ahead (the archdiff model page
// "Qwen3.8-2.4T-A95B", components list: multi-token-prediction modules and
// self-drafting speculative decoding); the target model then runs every
// drafted token through each layer.  For a GDN layer that is Tv steps of the
// gated delta rule (podcast transcript on "On the Design of Qwen3.8-Next
// Architecture", cue 14) from the state the sequence has reached, one per
// token, in the stored layout M = S^T:
//   r = M^T k_t, p = M^T q_t, u = beta_t (v_t - alpha_t r),
//   o_t = scale (alpha_t p + (k_t . q_t) u),  M <- alpha_t M + k_t u^T.
// A workgroup reads its dk x dv fp32 slice once, keeps it in registers for
// all Tv tokens and writes it once (and, on request, after every token, so a
// caller that accepts only a prefix of the draft can continue from the state
// after its last accepted token).  Like the single step it is bound by HBM
// bandwidth, with Tv times the tokens per state pass.
#include "device_common.hpp"
#include "launch.hpp"

namespace gdn {
namespace {

constexpr int kVerifyThreads = 256;

template <class T, int DK, int DV>
__global__ __launch_bounds__(kVerifyThreads) void verify_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const float* __restrict__ g,
    const float* __restrict__ beta, const float* state_in, float* state_out, float* __restrict__ token_states,
    T* __restrict__ o, int Tv, int Hqk, int Hv, float scale) {
  constexpr int TPR = DV / 4;                  // threads per state row (one float4 each)
  constexpr int RG = kVerifyThreads / TPR;     // row groups
  constexpr int RPT = DK / RG;                 // rows per thread: rg, rg + RG, ...
  constexpr int NWAVE = kVerifyThreads / 64;
  static_assert(DK % RG == 0 && 64 % TPR == 0, "shape");

  const int unit = blockIdx.x;  // n * Hv + h
  const int n = unit / Hv;
  const int h = unit - n * Hv;
  const int hq = h / (Hv / Hqk);
  const int tid = threadIdx.x;
  const int cg = tid % TPR;
  const int rg = tid / TPR;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  __shared__ float sk[kMaxVerifyTokens][DK];
  __shared__ float sq[kMaxVerifyTokens][DK];
  __shared__ float sv[kMaxVerifyTokens][DV];
  __shared__ float sab[kMaxVerifyTokens][2];        // alpha, beta per token
  __shared__ floatx4 red_r[2][NWAVE][TPR];          // by token parity: one barrier per token
  __shared__ floatx4 red_p[2][NWAVE][TPR];
  __shared__ float red_kq[2][NWAVE];

  // The state slice first: these loads dominate the run time.
  const size_t sbase = static_cast<size_t>(unit) * DK * DV;
  floatx4 m[RPT];
#pragma unroll
  for (int r = 0; r < RPT; ++r)
    m[r] = *reinterpret_cast<const floatx4*>(state_in + sbase + static_cast<size_t>(rg + RG * r) * DV + 4 * cg);

  // Every token's key, query, value and gates into LDS.
  for (int i = tid; i < Tv * DK; i += kVerifyThreads) {
    const int t = i / DK, c = i - t * DK;
    const size_t row = (static_cast<size_t>(n) * Tv + t) * Hqk + hq;
    sk[t][c] = to_float(k[row * DK + c]);
    sq[t][c] = to_float(q[row * DK + c]);
  }
  for (int i = tid; i < Tv * DV; i += kVerifyThreads) {
    const int t = i / DV, c = i - t * DV;
    sv[t][c] = to_float(v[((static_cast<size_t>(n) * Tv + t) * Hv + h) * DV + c]);
  }
  if (tid < Tv) {
    const size_t tu = (static_cast<size_t>(n) * Tv + tid) * Hv + h;
    sab[tid][0] = expf(g[tu]);
    sab[tid][1] = beta[tu];
  }
  __syncthreads();

  for (int t = 0; t < Tv; ++t) {
    const int par = t & 1;
    floatx4 r = zero4(), p = zero4();
    float kq = 0.f;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const float ki = sk[t][rg + RG * i], qi = sq[t][rg + RG * i];
      r += ki * m[i];
      p += qi * m[i];
      kq += ki * qi;
    }
    // Sum over the row groups inside the wavefront, then across wavefronts.
#pragma unroll
    for (int off = TPR; off < 64; off <<= 1) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        r[c] += __shfl_xor(r[c], off);
        p[c] += __shfl_xor(p[c], off);
      }
      kq += __shfl_xor(kq, off);
    }
    if (lane < TPR) {
      red_r[par][wave][cg] = r;
      red_p[par][wave][cg] = p;
      if (lane == 0) red_kq[par][wave] = kq;
    }
    __syncthreads();
    r = red_r[par][0][cg];
    p = red_p[par][0][cg];
    kq = red_kq[par][0];
#pragma unroll
    for (int w = 1; w < NWAVE; ++w) {
      r += red_r[par][w][cg];
      p += red_p[par][w][cg];
      kq += red_kq[par][w];
    }
    const float alpha = sab[t][0], b = sab[t][1];
    const floatx4 vv = *reinterpret_cast<const floatx4*>(&sv[t][4 * cg]);
    const floatx4 u = b * (vv - alpha * r);
#pragma unroll
    for (int i = 0; i < RPT; ++i) m[i] = alpha * m[i] + sk[t][rg + RG * i] * u;
    const size_t tu = (static_cast<size_t>(n) * Tv + t) * Hv + h;
    if (rg == 0) {
      const floatx4 ov = scale * (alpha * p + kq * u);
      *reinterpret_cast<typename Vec4<T>::type*>(o + tu * DV + 4 * cg) = pack4<T>(ov[0], ov[1], ov[2], ov[3]);
    }
    if (token_states) {
      float* ts = token_states + tu * DK * DV;
#pragma unroll
      for (int i = 0; i < RPT; ++i)
        __builtin_nontemporal_store(m[i], reinterpret_cast<floatx4*>(ts + static_cast<size_t>(rg + RG * i) * DV + 4 * cg));
    }
  }
  // Streaming stores: the state is not read again until the next call (as in
  // the single step).  Each thread writes back exactly the elements it read,
  // so state_out may be state_in.
  if (state_out) {
#pragma unroll
    for (int i = 0; i < RPT; ++i)
      __builtin_nontemporal_store(m[i], reinterpret_cast<floatx4*>(state_out + sbase +
                                                                    static_cast<size_t>(rg + RG * i) * DV + 4 * cg));
  }
}

template <class T, int DK, int DV>
hipError_t launch(const VerifyArgs& a, hipStream_t stream) {
  const int units = a.num_seqs * a.Hv;
  if (units == 0) return hipSuccess;
  verify_kernel<T, DK, DV><<<dim3(units), dim3(kVerifyThreads), 0, stream>>>(
      static_cast<const T*>(a.q), static_cast<const T*>(a.k), static_cast<const T*>(a.v), a.g, a.beta,
      a.state_in, a.state_out, a.token_states, static_cast<T*>(a.o), a.tokens, a.Hqk, a.Hv, a.scale);
  return hipGetLastError();
}

template <class T>
hipError_t dispatch_dims(const VerifyArgs& a, hipStream_t stream) {
  if (a.dk == 128 && a.dv == 128) return launch<T, 128, 128>(a, stream);
  if (a.dk == 64 && a.dv == 64) return launch<T, 64, 64>(a, stream);
  if (a.dk == 128 && a.dv == 64) return launch<T, 128, 64>(a, stream);
  if (a.dk == 64 && a.dv == 128) return launch<T, 64, 128>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_verify(const VerifyArgs& a, hipStream_t stream) {
  return a.bf16 ? dispatch_dims<bf16>(a, stream) : dispatch_dims<float>(a, stream);
}

}  // namespace gdn

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
#include "lane_sums.hpp"
#include "launch.hpp"

namespace gdn {
namespace {

constexpr int kVerifyThreads = 256;

// Each wavefront owns a block of DV / 4 state columns over all DK rows, so the
// reductions over the key dimension (M^T k, M^T q, k . q) stay inside the
// wavefront (DPP and row swaps, no LDS) and the token loop runs without a workgroup
// barrier.  A thread holds rows rg, rg + RG, ... of four columns, so a load
// instruction covers RG consecutive rows.
template <class T, int DK, int DV>
__global__ __launch_bounds__(kVerifyThreads) void verify_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const float* __restrict__ g,
    const float* __restrict__ beta, const float* state_in, float* state_out, float* __restrict__ token_states,
    T* __restrict__ o, int Tv, int Hqk, int Hv, float scale) {
  constexpr int NWAVE = kVerifyThreads / 64;
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

  __shared__ float sk[kMaxVerifyTokens][DK];
  __shared__ float sq[kMaxVerifyTokens][DK];
  __shared__ float sv[kMaxVerifyTokens][DV];
  __shared__ float sab[kMaxVerifyTokens][2];  // alpha, beta per token

  // The tokens' keys, queries and values first, as whole 16-byte pieces, one array per wavefront
  // (unconditional loads, clamped to the last piece); then the state slice, whose loads dominate the
  // run time; then the tokens into LDS, which waits only for the first loads, so that the barrier
  // and the first products overlap the state's arrival.
  constexpr int EPB = 16 / sizeof(T);  // elements per piece
  constexpr int PMAX = (kMaxVerifyTokens * (DK > DV ? DK : DV) / EPB + 63) / 64;  // pieces per lane
  typedef T piece_t __attribute__((ext_vector_type(16 / sizeof(T))));
  const int wave = tid >> 6;
  piece_t pc[PMAX];
  float gb = 0.f;
  {
    const int D = wave == 2 ? DV : DK, rowlen = D / EPB, np = Tv * rowlen;
#pragma unroll
    for (int i = 0; i < PMAX; ++i) {
      const int pi = min(lane + 64 * i, np - 1), t = pi / rowlen, e = (pi - t * rowlen) * EPB;
      const T* src = wave == 0 ? k + ((static_cast<size_t>(n) * Tv + t) * Hqk + hq) * DK + e
                   : wave == 1 ? q + ((static_cast<size_t>(n) * Tv + t) * Hqk + hq) * DK + e
                               : v + ((static_cast<size_t>(n) * Tv + t) * Hv + h) * DV + e;
      if (wave < 3) pc[i] = *reinterpret_cast<const piece_t*>(src);
    }
    if (wave == 3) {
      const size_t tu = (static_cast<size_t>(n) * Tv + min(lane >> 1, Tv - 1)) * Hv + h;
      gb = (lane & 1) ? beta[tu] : g[tu];
    }
  }
  const size_t sbase = static_cast<size_t>(unit) * DK * DV;
  floatx4 m[RPT];
#pragma unroll
  for (int r = 0; r < RPT; ++r)
    m[r] = *reinterpret_cast<const floatx4*>(state_in + sbase + static_cast<size_t>(rg + RG * r) * DV + col);
  {
    const int D = wave == 2 ? DV : DK, rowlen = D / EPB, np = Tv * rowlen;
    float* dst = wave == 0 ? &sk[0][0] : wave == 1 ? &sq[0][0] : &sv[0][0];
    const int ld = wave == 2 ? DV : DK;
    if (wave < 3) {
#pragma unroll
      for (int i = 0; i < PMAX; ++i) {
        const int pi = lane + 64 * i;
        if (pi < np) {
          const int t = pi / rowlen, e = (pi - t * rowlen) * EPB;
#pragma unroll
          for (int x = 0; x < EPB; ++x) dst[t * ld + e + x] = to_float(pc[i][x]);
        }
      }
    } else if (lane < 2 * Tv) {
      sab[lane >> 1][lane & 1] = (lane & 1) ? gb : expf(gb);
    }
  }
  __syncthreads();

  for (int t = 0; t < Tv; ++t) {
    floatx4 r = zero4(), p = zero4();
    float kq = 0.f;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const float ki = sk[t][rg + RG * i], qi = sq[t][rg + RG * i];
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
    const float alpha = sab[t][0], b = sab[t][1];
    const floatx4 vv = *reinterpret_cast<const floatx4*>(&sv[t][col]);
    const floatx4 u = b * (vv - alpha * r);
#pragma unroll
    for (int i = 0; i < RPT; ++i) m[i] = decay_write(m[i], alpha, sk[t][rg + RG * i], u);
    const size_t tu = (static_cast<size_t>(n) * Tv + t) * Hv + h;
    if (rg == 0) {
      const floatx4 ov = scale * (alpha * p + kq * u);
      *reinterpret_cast<typename Vec4<T>::type*>(o + tu * DV + col) = pack4<T>(ov[0], ov[1], ov[2], ov[3]);
    }
    if (token_states) {
      float* ts = token_states + tu * DK * DV;
#pragma unroll
      for (int i = 0; i < RPT; ++i)
        __builtin_nontemporal_store(m[i], reinterpret_cast<floatx4*>(ts + static_cast<size_t>(rg + RG * i) * DV + col));
    }
  }
  // Streaming stores: the state is not read again until the next call (as in
  // the single step).  Each thread writes back exactly the elements it read,
  // so state_out may be state_in.
  if (state_out) {
#pragma unroll
    for (int i = 0; i < RPT; ++i)
      __builtin_nontemporal_store(m[i], reinterpret_cast<floatx4*>(state_out + sbase +
                                                                    static_cast<size_t>(rg + RG * i) * DV + col));
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

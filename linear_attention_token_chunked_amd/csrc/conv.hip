// Pre-mixer step of the GDN layer: short causal convolution along the tokens,
// per channel, and (for q and k) an L2 normalisation of every head, gfx950.
//
// The podcast transcript on "On the Design of Qwen3.8-Next Architecture"
// (cue 14) lists short causal convolutions among what the model adds around
// the gated delta rule; it gives no width, and this library builds width 4.
// The archdiff model page "Qwen3.8-2.4T-A95B" normalises q and k per head
// (QK-Norm); here to unit L2 norm, the scale at which the delta rule's write
// with beta = 1 replaces exactly what is stored under a key.
// For channel c of token t of a sequence that starts at token s:
//   y[t, c] = sum_{i < W} w[c, i] * x[t - (W - 1) + i, c],   x[u] = 0 for u < s,
// then, with l2norm, y[t, head] /= sqrt(sum over the head's channels of y^2 + eps).
// The kernel is bound by HBM bandwidth: every token row is read once and
// written once.  Sixteen lanes share a (token, head) row of hd channels, so a
// row's norm reduces inside a 16-lane group.
#include "device_common.hpp"
#include "launch.hpp"

namespace gdn {
namespace {

constexpr int kConvThreads = 256;
constexpr int kConvWidth = 4;

// Sum over the 16 lanes of a DPP row, the same bits in every lane, without LDS: lanes i and 7 - i of
// each half-row (half-row mirror), then pairs l ^ 1 and l ^ 2 (quad permutations), then l ^ 8
// (rotation of the row by 8).
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

// A 16-lane group walks a run of kRun consecutive tokens of one head: it
// takes the head's taps from LDS (loaded once per workgroup) and slides a
// window of the last W token rows through registers.  A wavefront's four groups take four consecutive heads of
// one run, and the workgroup's four wavefronts take four consecutive runs of
// the same heads: a wavefront hands the last W - 1 rows of its run to the next
// one through LDS, so only the first run of a workgroup loads the rows before
// it again (3 of every 32 rows instead of 3 of every 8), and those it finds in
// its XCD's L2 (see the workgroup numbering in the kernel).
constexpr int kRun = 8;
constexpr int kWaves = kConvThreads / 64;

template <class T, int HD, bool L2>
__global__ __launch_bounds__(kConvThreads) void conv_kernel(const T* __restrict__ x, const float* __restrict__ w,
                                                            T* __restrict__ y, const int32_t* __restrict__ cu,
                                                            int num_seqs, int seqlen, int heads, int tokens,
                                                            int head_blocks, int token_blocks, float eps) {
  constexpr int EPL = HD / 16;  // channels per lane
  constexpr int W = kConvWidth;
  static_assert(W == 4, "one 16-byte load of taps per channel");
  typedef T lane_vec __attribute__((ext_vector_type(EPL)));
  __shared__ lane_vec handoff[kWaves][W - 1][64];  // a wavefront's last W - 1 rows, lane by lane
  __shared__ floatx4 stap[4 * HD];                   // the taps of the workgroup's four heads
  const int lane = threadIdx.x & 63, lane16 = lane & 15;
  // (made uniform, so that the search for the sequence start below runs on scalar loads)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // Workgroup -> (token block, head block).  With head_blocks dividing 8, workgroup ids 8 apart (one
  // XCD) take consecutive token blocks of one head block, so the rows before a block, which the block
  // before it loaded, are found in that XCD's L2; the 8 / head_blocks streams split the tokens in
  // equal parts.  Otherwise: token block id / head_blocks.
  int hb, tb;
  if (8 % head_blocks == 0) {
    const int x = blockIdx.x & 7, j = blockIdx.x >> 3, streams = 8 / head_blocks;
    hb = x % head_blocks;
    tb = j + (x / head_blocks) * ((token_blocks + streams - 1) / streams);
  } else {
    hb = blockIdx.x % head_blocks;
    tb = blockIdx.x / head_blocks;
  }
  if (tb >= token_blocks) return;  // (whole workgroups)
  const int h = hb * 4 + (lane >> 4);
  const bool active = h < heads;  // (inactive groups still take part in the barrier)
  const int t0 = tb * (kWaves * kRun) + wave * kRun;
  const int c0 = (active ? h : 0) * HD + lane16 * EPL;  // first channel of this lane
  // The taps of heads 4 hb .. 4 hb + 3, each channel's four loaded once per workgroup rather than once
  // per wavefront (unconditional loads, clamped to the last channel), and stored to LDS only after the
  // rows' loads are issued, so that the store's wait does not hold those back.
  constexpr int TPT = 4 * HD / kConvThreads;  // tap vectors per thread
  static_assert(4 * HD % kConvThreads == 0, "taps split evenly");
  floatx4 tapr[TPT];
#pragma unroll
  for (int j = 0; j < TPT; ++j)
    tapr[j] = *reinterpret_cast<const floatx4*>(
        w + static_cast<size_t>(min(hb * 4 * HD + static_cast<int>(threadIdx.x) + j * kConvThreads, heads * HD - 1)) * W);
  const T* xl = x + c0;  // this lane's channels of token 0
  T* yl = y + c0;
  const size_t tstride = static_cast<size_t>(heads) * HD;
  // the run's rows (past the last token, the last row again: never used)
  lane_vec rows[kRun];
#pragma unroll
  for (int r = 0; r < kRun; ++r)
    rows[r] = *reinterpret_cast<const lane_vec*>(xl + static_cast<size_t>(min(t0 + r, tokens - 1)) * tstride);
  // rows t0 - 3 .. t0 - 1: from the wavefront before (LDS) or, for the first, from memory
  lane_vec prev[W - 1];
  if (wave == 0) {
#pragma unroll
    for (int i = 0; i < W - 1; ++i)
      prev[i] = *reinterpret_cast<const lane_vec*>(xl + static_cast<size_t>(max(t0 - (W - 1) + i, 0)) * tstride);
  }
  // The sequence of the run's first token, and where the next one starts.  The search waits on each
  // of its reads, so it runs after the rows' loads are issued, on scalar loads (their own counter: it
  // does not wait for the rows).
  int start, next;
  if (cu) {
    int lo = 0, hi = num_seqs;  // the last n with cu[n] <= t0
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (cu[mid] <= t0) lo = mid; else hi = mid;
    }
    start = cu[lo];
    next = cu[lo + 1];  // > t0 unless t0 is past the last token
  } else {
    start = t0 - t0 % seqlen;
    next = start + seqlen;
  }
#pragma unroll
  for (int j = 0; j < TPT; ++j) stap[threadIdx.x + j * kConvThreads] = tapr[j];
#pragma unroll
  for (int i = 0; i < W - 1; ++i) handoff[wave][i][lane] = rows[kRun - (W - 1) + i];
  __syncthreads();
  floatx4 taps[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) taps[e] = stap[(lane >> 4) * HD + lane16 * EPL + e];
  if (wave > 0) {
#pragma unroll
    for (int i = 0; i < W - 1; ++i) prev[i] = handoff[wave - 1][i][lane];
  }
  if (!active || t0 >= tokens) return;
  // window of the W - 1 rows before the current token (zero before the sequence start)
  float win[W - 1][EPL];
#pragma unroll
  for (int i = 0; i < W - 1; ++i) {
    const int u = t0 - (W - 1) + i;
    const bool live = u >= start && u >= 0;
#pragma unroll
    for (int e = 0; e < EPL; ++e) win[i][e] = live ? to_float(prev[i][e]) : 0.f;
  }
#pragma unroll
  for (int r = 0; r < kRun; ++r) {
    const int t = t0 + r;
    if (t >= tokens) break;
    if (t == next) {  // a new sequence starts here: forget the window
      start = t;
      if (cu) {  // the last sequence starting at or before t (empty ones start and end at t)
        int lo = 0, hi = num_seqs;
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if (cu[mid] <= t) lo = mid; else hi = mid;
        }
        next = cu[lo + 1];
      } else {
        next = t + seqlen;
      }
#pragma unroll
      for (int i = 0; i < W - 1; ++i)
#pragma unroll
        for (int e = 0; e < EPL; ++e) win[i][e] = 0.f;
    }
    const lane_vec v = rows[r];
    float cur[EPL], acc[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      cur[e] = to_float(v[e]);
      acc[e] = taps[e][0] * win[0][e] + taps[e][1] * win[1][e] + taps[e][2] * win[2][e] + taps[e][3] * cur[e];
    }
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      win[0][e] = win[1][e];
      win[1][e] = win[2][e];
      win[2][e] = cur[e];
    }
    if constexpr (L2) {
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) ss += acc[e] * acc[e];
      const float rs = rsqrtf(row16_sum(ss) + eps);
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] *= rs;
    }
#pragma unroll
    for (int e = 0; e < EPL; e += 4)
      // (streaming stores: the rows are read again only by the mixer, after much else)
      __builtin_nontemporal_store(pack4<T>(acc[e], acc[e + 1], acc[e + 2], acc[e + 3]),
                                  reinterpret_cast<typename Vec4<T>::type*>(yl + static_cast<size_t>(t) * tstride + e));
  }
}

template <class T, int HD>
hipError_t launch(const ConvArgs& a, hipStream_t stream) {
  if (a.tokens == 0) return hipSuccess;
  const int head_blocks = (a.heads + 3) / 4;
  const int token_blocks = (a.tokens + kWaves * kRun - 1) / (kWaves * kRun);
  int64_t blocks = static_cast<int64_t>(token_blocks) * head_blocks;
  if (8 % head_blocks == 0) {  // (see the kernel: 8 / head_blocks token streams, 8 ids per step)
    const int streams = 8 / head_blocks;
    blocks = 8 * static_cast<int64_t>((token_blocks + streams - 1) / streams);
  }
  const dim3 grid(static_cast<unsigned>(blocks));
  if (a.l2norm)
    conv_kernel<T, HD, true><<<grid, dim3(kConvThreads), 0, stream>>>(
        static_cast<const T*>(a.x), a.weight, static_cast<T*>(a.y), a.cu_seqlens, a.num_seqs, a.seqlen, a.heads,
        a.tokens, head_blocks, token_blocks, a.eps);
  else
    conv_kernel<T, HD, false><<<grid, dim3(kConvThreads), 0, stream>>>(
        static_cast<const T*>(a.x), a.weight, static_cast<T*>(a.y), a.cu_seqlens, a.num_seqs, a.seqlen, a.heads,
        a.tokens, head_blocks, token_blocks, a.eps);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_conv(const ConvArgs& a, hipStream_t stream) {
  if (a.head_dim == 128) return a.bf16 ? launch<bf16, 128>(a, stream) : launch<float, 128>(a, stream);
  if (a.head_dim == 64) return a.bf16 ? launch<bf16, 64>(a, stream) : launch<float, 64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace gdn

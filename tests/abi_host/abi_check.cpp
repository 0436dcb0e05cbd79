// Host-only check of the C ABI's argument handling, built with AddressSanitizer and
// UndefinedBehaviorSanitizer together with the library's real validation (gdn_api.cpp) and
// workspace planning (plan.cpp).  The kernel launchers are replaced by stubs that record the
// arguments a call would launch with, so no GPU is needed: every call below either is rejected
// before any HIP call, or reaches a stub whose recorded arguments are checked.
//
// Pointers are aligned fake addresses that nothing here dereferences.  Extreme sizes (INT_MAX
// tokens, heads and sequences) exercise the 64-bit size arithmetic under the sanitizers.
// Exit status 0 and "abi_check ok" when every case holds.
#include <limits.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "gdn.h"
#include "launch.hpp"

extern "C" int c_caller_checks(void);  // abi_c_caller.c

namespace {

enum Kind { NONE, PREFILL, PREFILL_NOALLOC, DECODE, VERIFY, NORM_GATE, CONV, BWD };
Kind g_kind = NONE;
gdn::PrefillArgs g_prefill;
gdn::BwdArgs g_bwd;
int g_failures = 0, g_cases = 0;

void expect(bool ok, const char* what, int line) {
  ++g_cases;
  if (!ok) {
    ++g_failures;
    fprintf(stderr, "FAILED line %d: %s\n", line, what);
  }
}
#define EXPECT(x) expect((x), #x, __LINE__)

void* fake(uintptr_t off = 0) { return reinterpret_cast<void*>(uintptr_t(1) << 20 | off); }
float* ffake(uintptr_t off = 0) { return static_cast<float*>(fake(off)); }
const int32_t* ifake(uintptr_t off = 0) { return static_cast<const int32_t*>(fake(off)); }

gdn_dims_t dims(int B = 1, int T = 128, int N = 1, int Hqk = 2, int Hv = 4, int dk = 128, int dv = 128,
                int chunk = 64, gdn_dtype_t dt = GDN_DTYPE_BFLOAT16) {
  gdn_dims_t d;
  d.batch = B;
  d.seqlen = T;
  d.num_seqs = N;
  d.num_qk_heads = Hqk;
  d.num_v_heads = Hv;
  d.head_dim_k = dk;
  d.head_dim_v = dv;
  d.chunk_size = chunk;
  d.scale = 1.f;
  d.dtype = dt;
  return d;
}

gdn_status_t fwd(const gdn_dims_t* d, const int32_t* cu = nullptr, void* ws = nullptr, size_t wsb = 0,
                 void* q = fake(), float* g = ffake(), float* h0 = nullptr) {
  g_kind = NONE;
  return gdn_fwd_chunked(d, q, fake(), fake(), g, ffake(), h0, cu, fake(), ffake(), ws, wsb, nullptr);
}

gdn_status_t noalloc(const gdn_dims_t* d, const int32_t* cu = nullptr, void* q = fake()) {
  g_kind = NONE;
  return gdn_fwd_chunked_noalloc(d, q, fake(), fake(), ffake(), ffake(), nullptr, cu, fake(), ffake(), nullptr);
}

}  // namespace

// ---------------------------------------------------------------- recording launchers
namespace gdn {
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t) {
  g_kind = PREFILL;
  g_prefill = a;
  return hipSuccess;
}
hipError_t launch_prefill_noalloc(const PrefillArgs& a, hipStream_t) {
  g_kind = PREFILL_NOALLOC;
  g_prefill = a;
  return hipSuccess;
}
hipError_t launch_decode(const DecodeArgs&, hipStream_t) {
  g_kind = DECODE;
  return hipSuccess;
}
hipError_t launch_verify(const VerifyArgs&, hipStream_t) {
  g_kind = VERIFY;
  return hipSuccess;
}
hipError_t launch_norm_gate(const EpilogueArgs&, hipStream_t) {
  g_kind = NORM_GATE;
  return hipSuccess;
}
hipError_t launch_conv(const ConvArgs&, hipStream_t) {
  g_kind = CONV;
  return hipSuccess;
}
hipError_t launch_bwd(const BwdArgs& a, hipStream_t) {
  g_kind = BWD;
  g_bwd = a;
  return hipSuccess;
}
}  // namespace gdn

int main() {
  // status strings, including an unknown code
  for (int s = 0; s <= 6; ++s) EXPECT(strlen(gdn_status_string(static_cast<gdn_status_t>(s))) > 0);

  // ---- gdn_fwd_chunked
  EXPECT(gdn_fwd_chunked_workspace_size(nullptr) == 0);
  EXPECT(gdn_fwd_chunked(nullptr, fake(), fake(), fake(), ffake(), ffake(), nullptr, nullptr, fake(), nullptr,
                         nullptr, 0, nullptr) == GDN_STATUS_INVALID_VALUE);
  gdn_dims_t d = dims();
  EXPECT(fwd(&d) == GDN_STATUS_SUCCESS && g_kind == PREFILL && g_prefill.num_seqs == 1 && g_prefill.Hv == 4 &&
         g_prefill.bf16 && g_prefill.workspace == nullptr);
  d = dims(1, 128, 1, 2, 3);
  EXPECT(fwd(&d) == GDN_STATUS_INVALID_VALUE && g_kind == NONE);  // Hv not a multiple of Hqk
  d = dims(1, 128, 1, 0, 4);
  EXPECT(fwd(&d) == GDN_STATUS_INVALID_VALUE);
  d = dims(1, 128, 1, 2, 4, 32, 32);
  EXPECT(fwd(&d) == GDN_STATUS_NOT_SUPPORTED);
  d = dims(1, 128, 1, 2, 4, 128, 128, 32);
  EXPECT(fwd(&d) == GDN_STATUS_NOT_SUPPORTED);
  d = dims(1, 128, 1, 2, 4, 128, 64);
  EXPECT(fwd(&d) == GDN_STATUS_NOT_SUPPORTED);
  d = dims(1, 128, 1, 2, 4, 128, 128, 64, GDN_DTYPE_FLOAT32);
  EXPECT(fwd(&d) == GDN_STATUS_NOT_SUPPORTED);  // fp32 prefill is built for d = 64
  d = dims();
  {
    const int bad = 7;
    memcpy(&d.dtype, &bad, sizeof bad);
  }
  EXPECT(fwd(&d) == GDN_STATUS_INVALID_VALUE);
  d = dims(-1, 128, -1);
  EXPECT(fwd(&d) == GDN_STATUS_INVALID_VALUE);
  d = dims(2, 128, 3);
  EXPECT(fwd(&d) == GDN_STATUS_INVALID_VALUE);  // N != B without cu_seqlens
  d = dims(2, 128, 2);
  EXPECT(fwd(&d, ifake()) == GDN_STATUS_INVALID_VALUE);  // cu_seqlens with B != 1
  d = dims(1, 128, 1, 2, 8192);
  EXPECT(fwd(&d) == GDN_STATUS_NOT_SUPPORTED);  // more value heads than 32-bit row offsets allow
  d = dims();
  EXPECT(fwd(&d, nullptr, nullptr, 0, nullptr) == GDN_STATUS_INVALID_VALUE);
  EXPECT(fwd(&d, nullptr, nullptr, 0, fake(8)) == GDN_STATUS_MISALIGNED);
  EXPECT(fwd(&d, nullptr, nullptr, 0, fake(), ffake(2)) == GDN_STATUS_MISALIGNED);
  EXPECT(fwd(&d, nullptr, nullptr, 0, fake(), ffake(), ffake(4)) == GDN_STATUS_MISALIGNED);
  d = dims(0, 128, 0);
  EXPECT(fwd(&d) == GDN_STATUS_SUCCESS && g_kind == NONE);  // no sequences: nothing launched

  // packed sequences: the longest-first order in the workspace; N = 1 is the batch row
  d = dims(1, 1000, 64, 16, 128);
  const size_t need = gdn_fwd_chunked_workspace_size(&d);
  EXPECT(need == 256);
  EXPECT(fwd(&d, ifake(), nullptr, need) == GDN_STATUS_INVALID_VALUE);
  EXPECT(fwd(&d, ifake(), fake(), need - 1) == GDN_STATUS_WORKSPACE_TOO_SMALL);
  EXPECT(fwd(&d, ifake(), fake(128), need) == GDN_STATUS_MISALIGNED);
  EXPECT(fwd(&d, ifake(), fake(), need) == GDN_STATUS_SUCCESS && g_prefill.cu_seqlens == ifake() &&
         g_prefill.workspace == fake() && g_prefill.workspace_bytes == need);
  d = dims(1, 65536, 1, 16, 32);
  const size_t seg = gdn_fwd_chunked_workspace_size(&d);
  EXPECT(seg > (size_t(1) << 29));
  EXPECT(fwd(&d, ifake(), fake(), seg) == GDN_STATUS_SUCCESS && g_prefill.cu_seqlens == nullptr);
  EXPECT(fwd(&d, nullptr, nullptr, seg) == GDN_STATUS_INVALID_VALUE);

  // extreme sizes: the size arithmetic is 64-bit, and token counts beyond 32-bit indices are refused
  d = dims(1, INT_MAX, 1, 1, 1);
  (void)gdn_fwd_chunked_workspace_size(&d);
  EXPECT(fwd(&d, nullptr, fake(), SIZE_MAX) == GDN_STATUS_NOT_SUPPORTED);
  d = dims(1, INT_MAX - 255, 1, 1, 1);
  EXPECT(fwd(&d, nullptr, fake(), SIZE_MAX) == GDN_STATUS_NOT_SUPPORTED);
  d = dims(1, INT_MAX - 256, 1, 1, 1);
  EXPECT(fwd(&d, nullptr, fake(), SIZE_MAX) == GDN_STATUS_SUCCESS);
  d = dims(INT_MAX, INT_MAX, INT_MAX, 4096, 4096);
  (void)gdn_fwd_chunked_workspace_size(&d);
  EXPECT(fwd(&d, nullptr, fake(), SIZE_MAX) == GDN_STATUS_NOT_SUPPORTED);
  d = dims(1, INT_MAX, INT_MAX, 1, 1);
  (void)gdn_fwd_chunked_workspace_size(&d);
  d = dims(1, 4096, 1, 1, 2);
  for (int T : {0, 1, 63, 64, 3071, 3072, 5000, 65536, INT_MAX - 64, INT_MAX}) {
    d.seqlen = T;
    (void)gdn_fwd_chunked_workspace_size(&d);
  }

  // ---- gdn_fwd_chunked_noalloc
  d = dims(1, 1000, 64, 16, 128);
  EXPECT(noalloc(&d, ifake()) == GDN_STATUS_SUCCESS && g_kind == PREFILL_NOALLOC && g_prefill.workspace == nullptr);
  d = dims(1, 9000, 4097, 1, 1);
  EXPECT(noalloc(&d, ifake()) == GDN_STATUS_WORKSPACE_TOO_SMALL && g_kind == NONE);
  d = dims(1, 9000, 4096, 1, 1);
  EXPECT(noalloc(&d, ifake()) == GDN_STATUS_SUCCESS);
  d = dims(1, 128, 1, 2, 3);
  EXPECT(noalloc(&d) == GDN_STATUS_INVALID_VALUE);
  d = dims();
  EXPECT(noalloc(&d, nullptr, fake(8)) == GDN_STATUS_MISALIGNED);
  d = dims(1, 4096, 1, 1, 2);
  EXPECT(noalloc(&d, ifake()) == GDN_STATUS_SUCCESS && g_prefill.cu_seqlens == nullptr);

  // ---- gdn_decode_step
  auto dec = [&](const gdn_dims_t* dd, float* state) {
    g_kind = NONE;
    return gdn_decode_step(dd, fake(), fake(), fake(), ffake(), ffake(), state, fake(), nullptr);
  };
  d = dims(256, 1, 256, 16, 32);
  EXPECT(dec(&d, ffake()) == GDN_STATUS_SUCCESS && g_kind == DECODE);
  EXPECT(dec(&d, nullptr) == GDN_STATUS_INVALID_VALUE);
  EXPECT(dec(&d, ffake(4)) == GDN_STATUS_MISALIGNED);
  d.seqlen = 2;
  EXPECT(dec(&d, ffake()) == GDN_STATUS_INVALID_VALUE);
  d = dims(INT_MAX, 1, INT_MAX, 1, 1);
  EXPECT(dec(&d, ffake()) == GDN_STATUS_SUCCESS);  // N * Hv < 2^31
  d = dims(INT_MAX, 1, INT_MAX, 2, 2);
  EXPECT(dec(&d, ffake()) == GDN_STATUS_NOT_SUPPORTED);

  // ---- gdn_decode_verify
  auto ver = [&](const gdn_dims_t* dd, float* state_out) {
    g_kind = NONE;
    return gdn_decode_verify(dd, fake(), fake(), fake(), ffake(), ffake(), ffake(), state_out, nullptr, fake(),
                             nullptr);
  };
  d = dims(256, 4, 256, 16, 32);
  EXPECT(ver(&d, nullptr) == GDN_STATUS_SUCCESS && g_kind == VERIFY);
  EXPECT(ver(&d, ffake(8)) == GDN_STATUS_MISALIGNED);
  d.seqlen = 9;
  EXPECT(ver(&d, nullptr) == GDN_STATUS_NOT_SUPPORTED);
  d.seqlen = 0;
  EXPECT(ver(&d, nullptr) == GDN_STATUS_INVALID_VALUE);

  // ---- gdn_output_norm_gate
  auto ng = [&](int64_t rows, int32_t dv, float eps, void* y) {
    g_kind = NONE;
    return gdn_output_norm_gate(rows, dv, eps, GDN_DTYPE_BFLOAT16, fake(), fake(), ffake(), y, nullptr);
  };
  EXPECT(ng(262144, 128, 1e-6f, fake()) == GDN_STATUS_SUCCESS && g_kind == NORM_GATE);
  EXPECT(ng(-1, 128, 1e-6f, fake()) == GDN_STATUS_INVALID_VALUE);
  EXPECT(ng(10, 96, 1e-6f, fake()) == GDN_STATUS_NOT_SUPPORTED);
  EXPECT(ng(10, 128, -1.f, fake()) == GDN_STATUS_INVALID_VALUE);
  EXPECT(ng(10, 128, 1e-6f, nullptr) == GDN_STATUS_INVALID_VALUE);
  EXPECT(ng(INT64_MAX, 128, 1e-6f, fake()) == GDN_STATUS_NOT_SUPPORTED);

  // ---- gdn_short_conv
  auto conv = [&](int B, int T, int N, const int32_t* cu, int heads, void* y) {
    g_kind = NONE;
    return gdn_short_conv(B, T, N, cu, heads, 128, 1, 1e-6f, GDN_DTYPE_BFLOAT16, fake(), ffake(), y, nullptr);
  };
  EXPECT(conv(4, 4096, 4, nullptr, 16, fake(1 << 12)) == GDN_STATUS_SUCCESS && g_kind == CONV);
  EXPECT(conv(4, 4096, 4, nullptr, 16, fake()) == GDN_STATUS_INVALID_VALUE);  // y == x
  EXPECT(conv(2, 100, 2, ifake(), 16, fake(1 << 12)) == GDN_STATUS_INVALID_VALUE);
  EXPECT(conv(1, INT_MAX, 1, nullptr, INT_MAX, fake(1 << 12)) == GDN_STATUS_NOT_SUPPORTED);

  // ---- gdn_bwd_chunked
  auto bwd = [&](const gdn_dims_t* dd, const int32_t* cu, void* ws, size_t wsb) {
    g_kind = NONE;
    return gdn_bwd_chunked(dd, fake(), fake(), fake(), ffake(), ffake(), nullptr, cu, fake(), nullptr, ffake(),
                           ffake(), ffake(), ffake(), ffake(), nullptr, ws, wsb, nullptr);
  };
  EXPECT(gdn_bwd_chunked_workspace_size(nullptr) == 0);
  d = dims(4, 4096, 4, 16, 16);
  const size_t bneed = gdn_bwd_chunked_workspace_size(&d);
  EXPECT(bneed > (size_t(1) << 28));
  EXPECT(bwd(&d, nullptr, fake(), bneed) == GDN_STATUS_SUCCESS && g_kind == BWD && g_bwd.workspace == fake());
  EXPECT(bwd(&d, nullptr, fake(), bneed - 1) == GDN_STATUS_WORKSPACE_TOO_SMALL);
  EXPECT(bwd(&d, nullptr, nullptr, bneed) == GDN_STATUS_INVALID_VALUE);
  EXPECT(bwd(&d, nullptr, fake(64), bneed) == GDN_STATUS_MISALIGNED);
  d = dims(INT_MAX, INT_MAX, INT_MAX, 4096, 4096);
  (void)gdn_bwd_chunked_workspace_size(&d);
  EXPECT(bwd(&d, nullptr, fake(), SIZE_MAX) == GDN_STATUS_NOT_SUPPORTED);

  const int c_failures = c_caller_checks();
  g_cases += 1;
  if (c_failures) {
    ++g_failures;
    fprintf(stderr, "FAILED: %d checks of the C caller\n", c_failures);
  }

  if (g_failures) {
    fprintf(stderr, "abi_check: %d of %d cases failed\n", g_failures, g_cases);
    return 1;
  }
  printf("abi_check ok: %d cases\n", g_cases);
  return 0;
}

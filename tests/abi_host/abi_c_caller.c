/* The C ABI called from C, where an enum object may hold any int: a dtype of 7 in gdn_dims_t or
 * as an argument must be rejected as GDN_STATUS_INVALID_VALUE without undefined behaviour in the
 * library (built with the sanitizers by tests/test_abi_sanitizers.py).  Returns the number of
 * failed checks. */
#include <stdint.h>

#include "gdn.h"

static void* fake(uintptr_t off) { return (void*)(((uintptr_t)1 << 20) | off); }

int c_caller_checks(void) {
  int failures = 0;
  gdn_dtype_t bad = (gdn_dtype_t)7;
  gdn_dims_t d = {1, 128, 1, 2, 4, 128, 128, 64, 1.0f, GDN_DTYPE_BFLOAT16};
  d.dtype = bad;
  failures += gdn_fwd_chunked_workspace_size(&d) != 0;
  failures += gdn_bwd_chunked_workspace_size(&d) == 0; /* sized as fp32: the call itself is rejected */
  failures += gdn_fwd_chunked(&d, fake(0), fake(0), fake(0), (const float*)fake(0), (const float*)fake(0), 0, 0,
                              fake(0), 0, 0, 0, 0) != GDN_STATUS_INVALID_VALUE;
  failures += gdn_fwd_chunked_noalloc(&d, fake(0), fake(0), fake(0), (const float*)fake(0), (const float*)fake(0),
                                      0, 0, fake(0), 0, 0) != GDN_STATUS_INVALID_VALUE;
  failures += gdn_decode_step(&d, fake(0), fake(0), fake(0), (const float*)fake(0), (const float*)fake(0),
                              (float*)fake(0), fake(0), 0) != GDN_STATUS_INVALID_VALUE;
  failures += gdn_output_norm_gate(10, 128, 1e-6f, bad, fake(0), fake(0), (const float*)fake(0), fake(0), 0) !=
              GDN_STATUS_INVALID_VALUE;
  failures += gdn_short_conv(1, 10, 1, 0, 1, 128, 0, 1e-6f, bad, fake(0), (const float*)fake(0), fake(4096), 0) !=
              GDN_STATUS_INVALID_VALUE;
  return failures;
}

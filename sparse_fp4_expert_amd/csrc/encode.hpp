// Device encoders of the FP4 (E2M1) values and E4M3 scales, shared by the
// weight packer and the activation quantizer.  Both take their decisions in
// fp32 (nearest, ties to the even code, saturating), as the format's
// definition and the CPU oracle do.
#pragma once

#include "common.hpp"

namespace moesq {

// E4M3 code of x >= 0: nearest, ties to even, saturating at 448.
__device__ __forceinline__ uint32_t e4m3_encode(float x) {
  if (!(x > 0.0f)) return 0;
  if (x >= 448.0f) return 0x7e;
  int ex;
  frexpf(x, &ex);                       // x = f * 2^ex, f in [0.5, 1)
  const int e = max(ex - 1, -6);        // floor(log2 x), subnormal range below 2^-6
  const float q = rintf(ldexpf(x, 3 - e));   // 3 fraction bits, exact scaling
  const int code = (e + 7) * 8 + (int)q - 8; // continuous across binades
  return (uint32_t)min(code, 0x7e);
}

// E2M1 code: nearest magnitude of {0,.5,1,1.5,2,3,4,6}, ties to even,
// saturating at 6; a zero magnitude is +0.
__device__ __forceinline__ uint32_t e2m1_encode(float q) {
  const float a = fabsf(q);
  uint32_t c;
  if (!(a < 6.0f)) {
    c = 7;
  } else if (a < 1.0f) {
    c = (uint32_t)rintf(a * 2.0f);                  // 0, 1 or 2
  } else {
    int ex;
    frexpf(a, &ex);
    const int e = ex - 1;                           // 0, 1 or 2
    const float m = rintf(ldexpf(a, 1 - e));        // 2, 3 or 4
    c = (uint32_t)((e + 1) * 2 + (int)m - 2);
  }
  if (q < 0.0f && c) c |= 8u;
  return c;
}

}  // namespace moesq

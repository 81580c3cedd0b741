// INT4 group quantiser shared by the encode kernels.
//
// NanoKV pages, Figure 4(b): residual coefficients are stored as INT4.  The
// format read here: a group is `g` consecutive coefficients of one token;
// scale = fp16 round-half-even of max|z|/7; code = clamp(rint(z/scale), -8, 7)
// with rint half-to-even; zero scale -> zero codes; two's-complement nibbles,
// coefficient 2j in the low nibble of byte j.
#pragma once

#include <hip/hip_fp16.h>

#include "nkv_common.hpp"

namespace nkv {

// z: g fp32 coefficients (any address space readable by the thread).
// Writes g/2 packed bytes to `codes` and the fp16 scale bits to `*scale`.
template <typename ZPtr>
__device__ __forceinline__ void quantize_group(ZPtr z, int g, uint8_t* codes,
                                               uint16_t* scale) {
  float m = 0.f;
  for (int j = 0; j < g; ++j) m = fmaxf(m, fabsf(z[j]));
  const float u = m / 7.0f;  // IEEE division (correctly rounded)
  const __half s = __float2half_rn(u);
  const float sf = __half2float(s);
  *scale = __half_as_ushort(s);
  for (int j = 0; j < g; j += 2) {
    int c0 = 0, c1 = 0;
    if (sf > 0.f) {
      c0 = (int)fminf(7.f, fmaxf(-8.f, rintf(z[j] / sf)));
      c1 = (int)fminf(7.f, fmaxf(-8.f, rintf(z[j + 1] / sf)));
    }
    codes[j >> 1] = uint8_t((c0 & 15) | ((c1 & 15) << 4));
  }
}

}  // namespace nkv

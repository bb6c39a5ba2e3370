// Block-scale encoders shared by the MX quantizer kernels and the W13
// epilogue that quantizes h2 rows (see mx.hip for the scale rule).
#pragma once

#include "common.h"

namespace moe {

__device__ __forceinline__ int e8m0_exp(float amax) {
  if (!(amax > 0.0f)) return -127;
  int p;
  const float m = frexpf(amax, &p);  // amax = m * 2^p, m in [0.5, 1); 448 = 0.875 * 2^9
  const int e = m <= 0.875f ? p - 9 : p - 8;
  return min(127, max(-127, e));
}

// E4M3 byte of v (|v| <= 448 after scaling; larger magnitudes saturate).
__device__ __forceinline__ uint32_t e4m3_rne(float v) {
  const uint32_t bits = __float_as_uint(v);
  const uint32_t sign = (bits >> 24) & 0x80u;
  float a = fminf(fabsf(v), 448.0f);
  uint32_t code;
  if (a < 0.015625f) {                       // below 2^-6: subnormal step 2^-9
    code = uint32_t(__builtin_rintf(a * 512.0f));  // 8 -> smallest normal, also right
  } else {
    const uint32_t ab = __float_as_uint(a);
    int E = int(ab >> 23) - 127;             // -6 .. 8
    uint32_t man = ab & 0x7fffffu;
    // round the 23-bit mantissa to 3 bits, ties to even
    const uint32_t lsb = (man >> 20) & 1u;
    man += 0x7ffffu + lsb;
    if (man & 0x800000u) {                   // carried into the exponent
      man = 0;
      E += 1;
    }
    code = (uint32_t(E + 7) << 3) | (man >> 20);
    code = min(code, 0x7eu);                 // 448 is the top (only reachable by rounding)
  }
  return sign | code;
}

__device__ __forceinline__ float ldexp_i(float v, int e) { return ldexpf(v, e); }

// MXFP4 (OCP MX E2M1 with E8M0 block scales): e = the smallest integer with
// amax <= 6 * 2^e, clamped to [-127, 127] (-127 for an all-zero block).
__device__ __forceinline__ int e8m0_exp_fp4(float amax) {
  if (!(amax > 0.0f)) return -127;
  int p;
  const float m = frexpf(amax, &p);  // 6 = 0.75 * 2^3
  const int e = m <= 0.75f ? p - 3 : p - 2;
  return min(127, max(-127, e));
}

// E2M1 code of v (bias 1: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6), nearest,
// ties to the even code; magnitudes above 6 saturate.  The grid spacing is
// 0.5 below 2, 1 in [2, 4) and 2 above, and every binade edge lies on the
// grid, so rounding a / spacing to the nearest even integer rounds to the
// grid (both scalings are exact).
__device__ __forceinline__ uint32_t e2m1_rne(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 28) & 8u;
  const float a = fminf(fabsf(v), 6.0f);
  float q;
  uint32_t code;
  if (a < 2.0f) {
    q = __builtin_rintf(a * 2.0f);            // 0..4 half-units
    code = uint32_t(q);                       // 0, 0.5, 1, 1.5 -> codes 0..3; 2.0 -> 4
  } else if (a < 4.0f) {
    q = __builtin_rintf(a);                   // 2..4
    code = uint32_t(q) + 2u;                  // 2 -> 4, 3 -> 5, 4 -> 6
  } else {
    q = __builtin_rintf(a * 0.5f);            // 2..3
    code = uint32_t(q) + 4u;                  // 4 -> 6, 6 -> 7
  }
  return sign | code;
}

}  // namespace moe

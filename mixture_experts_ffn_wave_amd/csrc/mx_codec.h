// MX-fp8 block codec shared by the quantisers and the GEMM epilogues that
// emit quantised operands: the UE8M0 block scale and the e4m3 conversion.
//
// KohakUwULLM README, "Key features": MXFP8 experts (e4m3 values, one
// power-of-two scale per 32 elements).  The scale is the smallest 2^x with
// amax <= 448 * 2^x, so nothing saturates; x is clamped to [-127, 127] and an
// all-zero block gets x = -127.

#pragma once

#include "common.h"

namespace moe {

// smallest x with amax <= 448 * 2^x, clamped to [-127, 127]
__device__ __forceinline__ int mx_scale_exp(float amax) {
  if (!(amax > 0.0f)) return -127;
  int e;
  const float m = frexpf(amax, &e);          // amax = (2m) 2^(e-1), 2m in [1, 2); 448 = 1.75 * 2^8
  const int x = (2.0f * m <= 1.75f) ? (e - 1) - 8 : (e - 1) - 7;
  return x < -127 ? -127 : (x > 127 ? 127 : x);
}

// Four scaled values (|v| * 2^-x <= 448, so nothing saturates) to four e4m3
// bytes, lowest first, with the hardware conversion (round to nearest even,
// e4m3 subnormals).  Scaling by 2^-x is exact: for a 16-bit input x <= 120,
// so 2^-x is a normal f32.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d, float s) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a * s, b * s, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c * s, d * s, w, true);
  return (uint32_t)w;
}

}  // namespace moe

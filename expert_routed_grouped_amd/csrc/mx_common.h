// MXFP8 helpers shared by the quantisation kernel and the W8A8 grouped FFN.
//
// MXFP8 (OCP microscaling, the format of the "Quantization" section of "Hosting
// Qwen on Blackwell"): 32 consecutive values along the contraction axis share
// one E8M0 scale byte s (value 2^(s-127)); each value is an OCP E4M3 code.
// Block rule used here: s = clamp(floor(log2 amax) - 8 + 127, 0, 254) (s = 0 for
// an all-zero block), code = E4M3 nearest to v / 2^(s-127), ties to even,
// magnitudes >= 448 saturate to 448, sign bit kept.
#pragma once
#include "common.h"

// E8M0 scale byte of a block whose largest magnitude is amax (finite, >= 0): the
// fp32 exponent field ef gives floor(log2 amax) = ef - 127 for normal amax, and
// ef - 8 <= 0 covers zero, subnormal and tiny blocks.
__device__ __forceinline__ uint32_t mx_scale_of(float amax) {
  const int ef = (int)((__float_as_uint(amax) >> 23) & 0xFF);
  return (uint32_t)max(ef - 8, 0);
}

// E4M3 code of a finite fp32 value: round to nearest, ties to the even code,
// saturating at 448, sign bit kept.
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fabsf(v);
  uint32_t mag;
  if (a >= 448.0f) {
    mag = 0x7Eu;
  } else if (a < 0.015625f) {  // below 2^-6: multiples of 2^-9 (code 8 is 2^-6 itself)
    mag = (uint32_t)__builtin_rintf(a * 512.0f);
  } else {  // 2^e * (1 + q/8), e in [-6, 8]; q == 8 carries into the exponent field
    const uint32_t bits = __float_as_uint(a);
    const int e = (int)(bits >> 23) - 127;
    const float m = __uint_as_float((bits & 0x7FFFFFu) | 0x3F800000u);
    const uint32_t q = (uint32_t)__builtin_rintf((m - 1.0f) * 8.0f);
    mag = ((uint32_t)(e + 7) << 3) + q;
  }
  return sign | mag;
}

// Largest magnitude over the 32 lanes of this half-wave (lanes 0-31 or 32-63).
__device__ __forceinline__ float halfwave_amax(float v) {
  float a = fabsf(v);
#pragma unroll
  for (int off = 16; off > 0; off >>= 1) a = fmaxf(a, __shfl_xor(a, off, 64));
  return a;
}

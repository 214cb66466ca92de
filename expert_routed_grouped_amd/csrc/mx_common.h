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

#include <type_traits>

// E8M0 scale byte of a block whose largest magnitude is amax (finite, >= 0): the
// fp32 exponent field ef gives floor(log2 amax) = ef - 127 for normal amax, and
// ef - 8 <= 0 covers zero, subnormal and tiny blocks.
__device__ __forceinline__ uint32_t mx_scale_of(float amax) {
  const int ef = (int)((__float_as_uint(amax) >> 23) & 0xFF);
  return (uint32_t)max(ef - 8, 0);
}

// E4M3 code of a finite fp32 value: round to nearest, ties to the even code,
// saturating at 448, sign bit kept.  The gfx950 packed conversion to OCP E4M3
// rounds to nearest even; clamping to +-448 first gives the saturation (checked
// on the GPU against a bit-by-bit encoder of the same rule over every E4M3 value,
// every midpoint between neighbours and one fp32 ulp either side of it, the
// saturation range and 4 M log-uniform random values: no difference).
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
  const float c = fminf(fmaxf(v, -448.0f), 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, 0.0f, 0, false) & 0xFFu;
}

// Largest magnitude over the 32 lanes of this half-wave (lanes 0-31 or 32-63), in every lane of
// it: DPP butterflies inside each row of 16 lanes (quad swaps, then the mirrored half row, then
// the mirrored row), then one exchange between the two rows.  Every lane must take part.
__device__ __forceinline__ float halfwave_amax(float v) {
  auto dpp = [](float x, auto CTRL) __attribute__((always_inline)) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), decltype(CTRL)::value, 0xf, 0xf, true));
  };
  float a = fabsf(v);
  a = fmaxf(a, dpp(a, std::integral_constant<int, 0xB1>{}));   // quad_perm [1, 0, 3, 2]
  a = fmaxf(a, dpp(a, std::integral_constant<int, 0x4E>{}));   // quad_perm [2, 3, 0, 1]
  a = fmaxf(a, dpp(a, std::integral_constant<int, 0x141>{}));  // row_half_mirror
  a = fmaxf(a, dpp(a, std::integral_constant<int, 0x140>{}));  // row_mirror
  return fmaxf(a, __shfl_xor(a, 16, 64));
}

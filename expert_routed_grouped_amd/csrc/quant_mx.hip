// moe_quantize_mx: rows x K (fp32 or bf16) -> MXFP8 codes [rows, K] and E8M0
// scales [rows, K/32].  Each lane takes 8 consecutive values (one 16-byte bf16
// load, or two for fp32) and four neighbouring lanes one block of 32: the block
// maximum needs two cross-lane steps, every lane writes its 8 codes as one
// 8-byte store and the first lane of the four the scale byte.  A grid-stride
// loop keeps every lane busy with several blocks.
#include "mx_common.h"

namespace {

template <bool BF16>
__global__ __launch_bounds__(256) void quantize_mx_kernel(const void *__restrict__ x, long long nvec,
                                                          uint8_t *__restrict__ codes, uint8_t *__restrict__ scales) {
  // nvec = elements / 8 is a multiple of 4, and so is the stride: the four lanes of a block
  // are always in the loop together
  const long long stride = (long long)gridDim.x * blockDim.x;
  for (long long v = (long long)blockIdx.x * blockDim.x + threadIdx.x; v < nvec; v += stride) {
    float f[8];
    if constexpr (BF16) {
      const u32x4_t q = *((const u32x4_t *)x + v);
      f[0] = bf16_lo(q.x); f[1] = bf16_hi(q.x); f[2] = bf16_lo(q.y); f[3] = bf16_hi(q.y);
      f[4] = bf16_lo(q.z); f[5] = bf16_hi(q.z); f[6] = bf16_lo(q.w); f[7] = bf16_hi(q.w);
    } else {
      const f32x4_t a = *((const f32x4_t *)x + 2 * v), b = *((const f32x4_t *)x + 2 * v + 1);
      f[0] = a[0]; f[1] = a[1]; f[2] = a[2]; f[3] = a[3]; f[4] = b[0]; f[5] = b[1]; f[6] = b[2]; f[7] = b[3];
    }
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; j++) amax = fmaxf(amax, fabsf(f[j]));
    amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
    const uint32_t s = mx_scale_of(amax);
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      lo |= e4m3_encode(ldexpf(f[j], 127 - (int)s)) << (8 * j);
      hi |= e4m3_encode(ldexpf(f[4 + j], 127 - (int)s)) << (8 * j);
    }
    *((uint2 *)codes + v) = make_uint2(lo, hi);
    if ((v & 3) == 0) scales[v >> 2] = (uint8_t)s;
  }
}

}  // namespace

hipError_t launch_quantize_mx(const void *x, int x_bf16, int rows, int K, uint8_t *codes, uint8_t *scales,
                              hipStream_t s) {
  const long long nvec = (long long)rows * K / 8;  // K % 32 == 0
  if (nvec == 0) return hipSuccess;
  const long long blocks = (nvec + 255) / 256;
  const unsigned grid = (unsigned)(blocks < 4096 ? blocks : 4096);
  if (x_bf16)
    hipLaunchKernelGGL(quantize_mx_kernel<true>, dim3(grid), dim3(256), 0, s, x, nvec, codes, scales);
  else
    hipLaunchKernelGGL(quantize_mx_kernel<false>, dim3(grid), dim3(256), 0, s, x, nvec, codes, scales);
  return hipGetLastError();
}

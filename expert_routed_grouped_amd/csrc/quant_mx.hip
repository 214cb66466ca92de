// moe_quantize_mx: rows x K (fp32 or bf16) -> MXFP8 codes [rows, K] and E8M0
// scales [rows, K/32].  One half-wave per block of 32: each lane loads one value,
// the block maximum comes from five cross-lane steps, every lane writes its code
// and the first lane of the half-wave the scale.
#include "mx_common.h"

namespace {

template <bool BF16>
__global__ __launch_bounds__(256) void quantize_mx_kernel(const void *__restrict__ x, long long nblocks, int kb,
                                                          uint8_t *__restrict__ codes, uint8_t *__restrict__ scales) {
  const long long g = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long blk = g >> 5;  // the 32 lanes of a half-wave share one block
  if (blk >= nblocks) return;    // nblocks * 32 threads: a half-wave is all in or all out
  const int i = (int)(g & 31);
  const long long idx = blk * 32 + i;
  const float v = BF16 ? bf16_to_f32(((const uint16_t *)x)[idx]) : ((const float *)x)[idx];
  const uint32_t s = mx_scale_of(halfwave_amax(v));
  codes[idx] = (uint8_t)e4m3_encode(ldexpf(v, 127 - (int)s));
  if (i == 0) scales[blk] = (uint8_t)s;
  (void)kb;
}

}  // namespace

hipError_t launch_quantize_mx(const void *x, int x_bf16, int rows, int K, uint8_t *codes, uint8_t *scales,
                              hipStream_t s) {
  const long long nblocks = (long long)rows * (K / 32);
  if (nblocks == 0) return hipSuccess;
  const long long threads = nblocks * 32;
  const unsigned grid = (unsigned)((threads + 255) / 256);
  if (x_bf16)
    hipLaunchKernelGGL(quantize_mx_kernel<true>, dim3(grid), dim3(256), 0, s, x, nblocks, K / 32, codes, scales);
  else
    hipLaunchKernelGGL(quantize_mx_kernel<false>, dim3(grid), dim3(256), 0, s, x, nblocks, K / 32, codes, scales);
  return hipGetLastError();
}

// Combine (moe_combine): y[t] = sum_j gate[t,j] * y_perm[token_row[t,j]], the
// weighted accumulation of "Hosting Qwen on Blackwell" (section "MoE Dispatch -
// Combine") and the routing-weighted sum of the AI-infra book, section 9.3.4.
// A pure streaming gather-reduce: one workgroup per token walks the k rows of
// that token in increasing j (a fixed order, so the result is deterministic)
// with 16-byte loads; the per-token indices and gates are wave-uniform.
#include "common.h"

namespace {

__global__ __launch_bounds__(256) void combine_kernel(const float4 *__restrict__ y_perm,
                                                      const int32_t *__restrict__ token_row,
                                                      const float *__restrict__ w, int T, int k, int H4,
                                                      float4 *__restrict__ y) {
  for (int t = blockIdx.x; t < T; t += gridDim.x) {
    for (int n = threadIdx.x; n < H4; n += blockDim.x) {
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int j = 0; j < k; j++) {
        const int r = token_row[(size_t)t * k + j];
        if (r < 0) continue;
        const float g = w[(size_t)t * k + j];
        const float4 v = y_perm[(size_t)r * H4 + n];
        acc.x = __builtin_fmaf(g, v.x, acc.x);
        acc.y = __builtin_fmaf(g, v.y, acc.y);
        acc.z = __builtin_fmaf(g, v.z, acc.z);
        acc.w = __builtin_fmaf(g, v.w, acc.w);
      }
      y[(size_t)t * H4 + n] = acc;
    }
  }
}

__global__ __launch_bounds__(256) void zero_kernel(float4 *__restrict__ p, size_t n4, float *__restrict__ tail,
                                                   int ntail) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride)
    p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  if (blockIdx.x == 0 && (int)threadIdx.x < ntail) tail[threadIdx.x] = 0.f;
}

}  // namespace

hipError_t launch_combine(const float *y_perm, const int32_t *token_row, const float *w, int T, int k, int H, float *y,
                          hipStream_t s) {
  if (T == 0) return hipSuccess;
  int grid = T < 16384 ? T : 16384;
  hipLaunchKernelGGL(combine_kernel, dim3(grid), dim3(256), 0, s, (const float4 *)y_perm, token_row, w, T, k, H / 4,
                     (float4 *)y);
  return hipGetLastError();
}

// Fill kernel rather than hipMemsetAsync, so a caller may capture it in a graph.
hipError_t launch_zero_f32(float *p, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  size_t n4 = n / 4;
  int ntail = (int)(n - n4 * 4);
  size_t blocks = (n4 + 255) / 256;
  int grid = (int)(blocks < 4096 ? (blocks ? blocks : 1) : 4096);
  hipLaunchKernelGGL(zero_kernel, dim3(grid), dim3(256), 0, s, (float4 *)p, n4, p + n4 * 4, ntail);
  return hipGetLastError();
}

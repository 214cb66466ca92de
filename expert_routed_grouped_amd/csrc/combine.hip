// Combine (moe_combine): y[t] = sum_j gate[t,j] * y_perm[token_row[t,j]], the
// weighted accumulation of "Hosting Qwen on Blackwell" (section "MoE Dispatch -
// Combine") and the routing-weighted sum of the AI-infra book, section 9.3.4.
// A pure streaming gather-reduce: one workgroup per token walks the k rows of
// that token in increasing j (a fixed order, so the result is deterministic)
// with 16-byte loads; the per-token indices and gates are wave-uniform.  For
// k <= 8 the loop over j has no branches: a dropped slot (row -1) reads one of
// the token's valid rows with gate 0, so all k loads of a column are in flight
// together.
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

template <int KMAX>
__global__ __launch_bounds__(256) void combine_k_kernel(const float4 *__restrict__ y_perm,
                                                        const int32_t *__restrict__ token_row,
                                                        const float *__restrict__ w, int T, int k, int H4,
                                                        float4 *__restrict__ y) {
  for (int t = blockIdx.x; t < T; t += gridDim.x) {
    int rr[KMAX];
    float gg[KMAX];
    int first = -1;
#pragma unroll
    for (int j = 0; j < KMAX; j++) {
      rr[j] = j < k ? token_row[(size_t)t * k + j] : -1;
      gg[j] = j < k ? w[(size_t)t * k + j] : 0.0f;
      if (first < 0 && rr[j] >= 0) first = rr[j];
    }
    if (first < 0) {  // no local slot: zeros
      for (int n = threadIdx.x; n < H4; n += blockDim.x) y[(size_t)t * H4 + n] = make_float4(0.f, 0.f, 0.f, 0.f);
      continue;
    }
#pragma unroll
    for (int j = 0; j < KMAX; j++) {
      if (rr[j] < 0) {
        rr[j] = first;
        gg[j] = 0.0f;
      }
    }
    const f32x4_t *src = (const f32x4_t *)y_perm;
    f32x4_t *dst = (f32x4_t *)y;
    for (int n = threadIdx.x; n < H4; n += blockDim.x) {
      f32x4_t v[KMAX];
#pragma unroll
      for (int j = 0; j < KMAX; j++) v[j] = __builtin_nontemporal_load(src + (size_t)rr[j] * H4 + n);
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < KMAX; j++) {
#pragma unroll
        for (int c = 0; c < 4; c++) acc[c] = __builtin_fmaf(gg[j], v[j][c], acc[c]);
      }
      __builtin_nontemporal_store(acc, dst + (size_t)t * H4 + n);
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
  if (k <= 8)
    hipLaunchKernelGGL(combine_k_kernel<8>, dim3(grid), dim3(256), 0, s, (const float4 *)y_perm, token_row, w, T, k,
                       H / 4, (float4 *)y);
  else
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

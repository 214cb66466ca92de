// Router GEMM + top-k + renormalised gates (moe_route).
//
// The router picks the top-K experts of every token (PagedAttention/MoE page,
// MoE list; AI-infra book, section 9.3.4).  The logit of (t, e) is an fp32
// fused-multiply-add chain over h in ascending order; this fixed order is the
// library's contract, so the chain is computed as is: one lane owns one expert
// and walks h upward, the token's activations are wave-uniform and come in
// through scalar loads.  Top-k is k rounds of a wave-wide max over 64-bit keys
// (orderable logit bits, inverted expert id), so equal logits go to the lower
// expert index; the gates are a softmax over the k selected logits.
#include "common.h"

namespace {

// Orderable key of an fp32 logit: larger float -> larger key, -0 mapped to +0.
__device__ __forceinline__ uint32_t ord_key(float v) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float ord_val(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    uint32_t lo = __shfl_xor((uint32_t)v, off, 64);
    uint32_t hi = __shfl_xor((uint32_t)(v >> 32), off, 64);
    uint64_t o = ((uint64_t)hi << 32) | lo;
    v = o > v ? o : v;
  }
  return v;
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Load 8 consecutive elements starting at p (16-byte aligned) as fp32.
template <bool BF16>
__device__ __forceinline__ void load8(const void *p, float (&f)[8]) {
  if constexpr (BF16) {
    uint4 v = *(const uint4 *)p;
    f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x); f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
    f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z); f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
  } else {
    float4 a = ((const float4 *)p)[0], b = ((const float4 *)p)[1];
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w; f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
  }
}

template <bool BF16>
__device__ __forceinline__ float load1(const void *p, size_t i) {
  if constexpr (BF16) return bf16_to_f32(((const uint16_t *)p)[i]);
  else return ((const float *)p)[i];
}

// Block = EC waves (wave c owns experts 64c .. 64c+63), TT tokens per block.
// VEC: H % 8 == 0 and 16-byte aligned rows (8-wide loads); otherwise one h at a time.
template <int TT, int EC, bool XB, bool WB, bool VEC>
__global__ __launch_bounds__(64 * EC) void route_kernel(const void *__restrict__ x, const void *__restrict__ w,
                                                        const float *__restrict__ bias, int T, int H, int E, int k,
                                                        int32_t *__restrict__ ids, float *__restrict__ gates) {
  __shared__ float lg[TT][64 * EC];
  const int lane = threadIdx.x & 63;
  const int c = threadIdx.x >> 6;
  const int e = c * 64 + lane;
  const bool ev = e < E;
  const int t0 = blockIdx.x * TT;
  const int esz_x = XB ? 2 : 4, esz_w = WB ? 2 : 4;
  const char *xrow[TT];
#pragma unroll
  for (int tt = 0; tt < TT; tt++) {
    int t = min(t0 + tt, T - 1);
    xrow[tt] = (const char *)x + (size_t)t * H * esz_x;
  }
  const char *wrow = (const char *)w + (size_t)(ev ? e : 0) * H * esz_w;

  float acc[TT];
#pragma unroll
  for (int tt = 0; tt < TT; tt++) acc[tt] = 0.0f;

  if constexpr (VEC) {
    for (int h = 0; h < H; h += 8) {
      float wf[8];
      load8<WB>(wrow + (size_t)h * esz_w, wf);
#pragma unroll
      for (int tt = 0; tt < TT; tt++) {
        float xf[8];
        load8<XB>(xrow[tt] + (size_t)h * esz_x, xf);
#pragma unroll
        for (int j = 0; j < 8; j++) acc[tt] = __builtin_fmaf(xf[j], wf[j], acc[tt]);
      }
    }
  } else {
    for (int h = 0; h < H; h++) {
      float wf = load1<WB>(wrow, h);
#pragma unroll
      for (int tt = 0; tt < TT; tt++) acc[tt] = __builtin_fmaf(load1<XB>(xrow[tt], h), wf, acc[tt]);
    }
  }
  if (bias != nullptr && ev) {
    float b = bias[e];
#pragma unroll
    for (int tt = 0; tt < TT; tt++) acc[tt] = acc[tt] + b;
  }
#pragma unroll
  for (int tt = 0; tt < TT; tt++) lg[tt][e] = acc[tt];
  __syncthreads();

  // top-k: wave c handles tokens c, c+EC, ...
  for (int tt = c; tt < TT; tt += EC) {
    const int t = t0 + tt;
    if (t >= T) break;
    uint64_t key[EC];
#pragma unroll
    for (int q = 0; q < EC; q++) {
      int eq = q * 64 + lane;
      key[q] = eq < E ? (((uint64_t)ord_key(lg[tt][eq]) << 32) | (uint32_t)~(uint32_t)eq) : 0ull;
    }
    float my_v = 0.0f, m = 0.0f;
    int my_e = 0;
    for (int j = 0; j < k; j++) {
      uint64_t best = key[0];
#pragma unroll
      for (int q = 1; q < EC; q++) best = key[q] > best ? key[q] : best;
      best = wave_max_u64(best);
      const int es = (int)~(uint32_t)best;
      const float vs = ord_val((uint32_t)(best >> 32));
#pragma unroll
      for (int q = 0; q < EC; q++)
        if (q * 64 + lane == es) key[q] = 0ull;
      if (j == 0) m = vs;
      if (lane == j) { my_v = vs; my_e = es; }
    }
    float u = lane < k ? expf(my_v - m) : 0.0f;
    float sum = wave_sum_f32(u);
    if (lane < k) {
      ids[(size_t)t * k + lane] = my_e;
      gates[(size_t)t * k + lane] = u / sum;
    }
  }
}

template <int TT, int EC>
hipError_t launch_tt(const void *x, int xb, const void *w, int wb, const float *bias, int T, int H, int E, int k,
                     int32_t *ids, float *gates, hipStream_t s) {
  dim3 grid(ceil_div_i(T, TT)), block(64 * EC);
  bool vec = (H % 8 == 0) && (((uintptr_t)x | (uintptr_t)w) % 16 == 0);
#define ROUTE_CASE(XB, WB, V)                                                                                 \
  if (xb == XB && wb == WB && vec == V) {                                                                   \
    hipLaunchKernelGGL((route_kernel<TT, EC, XB, WB, V>), grid, block, 0, s, x, w, bias, T, H, E, k, ids, gates); \
    return hipGetLastError();                                                                               \
  }
  ROUTE_CASE(true, true, true) ROUTE_CASE(true, true, false) ROUTE_CASE(false, false, true)
  ROUTE_CASE(false, false, false) ROUTE_CASE(true, false, true) ROUTE_CASE(true, false, false)
  ROUTE_CASE(false, true, true) ROUTE_CASE(false, true, false)
#undef ROUTE_CASE
  return hipErrorInvalidValue;
}

template <int EC>
hipError_t launch_ec(const void *x, int xb, const void *w, int wb, const float *bias, int T, int H, int E, int k,
                     int32_t *ids, float *gates, hipStream_t s) {
  // Few tokens: one token per block keeps every chain on its own wave (latency);
  // many tokens: four tokens per block amortise the weight loads.
  if (T <= 512) return launch_tt<1, EC>(x, xb, w, wb, bias, T, H, E, k, ids, gates, s);
  return launch_tt<4, EC>(x, xb, w, wb, bias, T, H, E, k, ids, gates, s);
}

}  // namespace

hipError_t launch_route(const void *x, int x_bf16, const void *w, int w_bf16, const float *bias, int T, int H, int E,
                        int k, int32_t *ids, float *gates, hipStream_t s) {
  if (T == 0) return hipSuccess;
  int ec = ceil_div_i(E, 64);
  switch (ec) {
    case 1: return launch_ec<1>(x, x_bf16, w, w_bf16, bias, T, H, E, k, ids, gates, s);
    case 2: return launch_ec<2>(x, x_bf16, w, w_bf16, bias, T, H, E, k, ids, gates, s);
    case 3:
    case 4: return launch_ec<4>(x, x_bf16, w, w_bf16, bias, T, H, E, k, ids, gates, s);
    default: return launch_ec<8>(x, x_bf16, w, w_bf16, bias, T, H, E, k, ids, gates, s);
  }
}

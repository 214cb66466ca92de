// Device side of the router (moe_route, moe_route_dispatch, the fused decode layer).
//
// The router picks the top-K experts of every token (PagedAttention/MoE page,
// MoE list; AI-infra book, section 9.3.4).  The logit of (t, e) is an fp32
// fused-multiply-add chain over h in ascending order; this fixed order is the
// library's contract, so the chain is computed as is: one lane owns one expert
// and walks h upward.  Top-k is k rounds of a wave-wide max (DPP) over 64-bit
// keys (orderable logit bits, inverted expert id), so equal logits go to the
// lower expert index; the gates are a softmax over the k selected logits.
#pragma once
#include "common.h"

namespace rt {

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

// Wave-wide reductions on DPP (data-parallel primitives: a VALU operand taken from another lane
// of the same row of 16, or broadcast from the last lane of the previous row or pair of rows).
// Row shifts by 1, 2, 4 and 8 leave in lane 15 of every row the reduction of that row; the row
// broadcasts of lanes 15 and 31 then carry it across rows, so lane 63 holds the reduction of the
// whole wave, which readlane makes wave-uniform.  A lane a shift leaves without a source reads 0,
// the identity of both the unsigned maximum and the sum.  No LDS traffic is involved.
enum : int { kDppShr1 = 0x111, kDppShr2 = 0x112, kDppShr4 = 0x114, kDppShr8 = 0x118, kDppBcast15 = 0x142,
             kDppBcast31 = 0x143 };

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppShr1, 0xf, 0xf, true));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppShr2, 0xf, 0xf, true));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppShr4, 0xf, 0xf, true));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppShr8, 0xf, 0xf, true));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppBcast15, 0xa, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppBcast31, 0xc, 0xf, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Largest 64-bit key of the wave: the largest high word, then the largest low word among the
// lanes that hold it (lexicographic, i.e. the unsigned 64-bit maximum).
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  const uint32_t hi = wave_max_u32((uint32_t)(v >> 32));
  const uint32_t lo = wave_max_u32((uint32_t)(v >> 32) == hi ? (uint32_t)v : 0u);
  return ((uint64_t)hi << 32) | lo;
}

template <int CTRL, int ROWS, bool BOUND>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROWS, 0xf, BOUND));
}

__device__ __forceinline__ float wave_sum_f32(float v) {
  v += dpp_f32<kDppShr1, 0xf, true>(v);
  v += dpp_f32<kDppShr2, 0xf, true>(v);
  v += dpp_f32<kDppShr4, 0xf, true>(v);
  v += dpp_f32<kDppShr8, 0xf, true>(v);
  v += dpp_f32<kDppBcast15, 0xa, false>(v);
  v += dpp_f32<kDppBcast31, 0xc, false>(v);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
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

#ifndef ROUTE_NS
#define ROUTE_NS 8
#endif

// Block = EC waves (wave c owns experts 64c .. 64c+63), TT tokens per block.
// VEC: H % 8 == 0 and 16-byte aligned rows (8-wide loads); otherwise one h at a time.
// WP (with VEC, fp32): the router weight in the layout of moe_pack_router, [H/4][E][4] fp32:
// the 16 bytes of h = 4j .. 4j+3 of expert e at (j E + e) 16, so the 64 lanes of a wave read
// 1 KB contiguously instead of 64 rows 4H bytes apart, and no element needs unpacking.
// t0: first token of the block.  The router weight is usually cold (the expert weights of the previous
// layer call streamed through L2 since), so the caller's blocks first touch its 128-byte lines
// between them: block touch_id of touch_n touches lines touch_id * blockDim + i (+ multiples of
// touch_n * blockDim), pulling the whole matrix into the caches in one round trip instead of block
// after block waiting on the same misses (touch_n = 0: no touch).  Blocks may have more than EC
// waves: the others only take part in the barriers.
// RING: depth of the weight-load ring for bf16 weights (fp32 weights use half as many slots).
template <int TT, int EC, bool XB, bool WB, bool VEC, bool WP = false, int RING = ROUTE_NS>
__device__ __forceinline__ void route_tokens(const void *__restrict__ x, const void *__restrict__ w,
                                             const float *__restrict__ bias, int T, int H, int E, int k,
                                             int32_t *__restrict__ ids, float *__restrict__ gates, int t0,
                                             int touch_id, int touch_n) {
  static_assert(!WP || (VEC && !WB), "the packed router weight is fp32, read 16 bytes at a time");
  __shared__ float lg[TT][64 * EC];
  const int lane = threadIdx.x & 63;
  const int c = threadIdx.x >> 6;
  const bool active = c < EC;  // wave-uniform
  const int e = c * 64 + lane;
  const bool ev = e < E;
  const int esz_x = XB ? 2 : 4, esz_w = WB ? 2 : 4;
  const char *xrow[TT];
#pragma unroll
  for (int tt = 0; tt < TT; tt++) {
    int t = min(t0 + tt, T - 1);
    xrow[tt] = (const char *)x + (size_t)t * H * esz_x;
  }
  const char *wrow = WP ? (const char *)w + (size_t)(ev ? e : 0) * 16 : (const char *)w + (size_t)(ev ? e : 0) * H * esz_w;
  const size_t wpstep = (size_t)E * 16;  // WP: bytes from one 4-wide h group to the next
  uint32_t touch = 0;
  if (touch_n > 0) {
    const size_t nlines = (size_t)E * H * esz_w / 128;  // whole lines only: never past the end
    const size_t nthreads = (size_t)touch_n * blockDim.x;
    for (size_t l = (size_t)touch_id * blockDim.x + threadIdx.x; l < nlines; l += nthreads)
      touch |= *(const volatile uint32_t *)((const char *)w + l * 128);
  }
  // VEC: the block's activation rows, staged once in LDS as fp32 ([TT][H], dynamic size)
  extern __shared__ __attribute__((aligned(16))) float xs[];
  if constexpr (VEC) {
    const int rp = H / 8;
    for (int i = threadIdx.x; i < TT * rp; i += blockDim.x) {
      const int tt = i / rp, hp = i - tt * rp;
      float f[8];
      load8<XB>(xrow[tt] + (size_t)hp * 8 * esz_x, f);
      *(f32x4_t *)(xs + tt * H + hp * 8) = f32x4_t{f[0], f[1], f[2], f[3]};
      *(f32x4_t *)(xs + tt * H + hp * 8 + 4) = f32x4_t{f[4], f[5], f[6], f[7]};
    }
    __syncthreads();
  }

  float acc[TT];
#pragma unroll
  for (int tt = 0; tt < TT; tt++) acc[tt] = 0.0f;

  if (!active) {
  } else if constexpr (VEC) {
    // 32 h per step; a ring of ROUTE_NS register sets keeps the weight pieces of
    // the next ROUTE_NS-1 steps in flight while a step computes (each lane reads
    // its own expert row, so only prefetch depth hides the L2 latency)
    // fp32 weights take twice the registers per step: half the ring depth
    constexpr int HS = 32, P = HS * (WB ? 2 : 4) / 16, NS = WB ? RING : RING / 2;
    const int nsteps = H / (HS * NS) * NS;  // whole rounds of the ring; the rest runs below
    u32x4_t ring[NS][P];
    auto wload = [&](u32x4_t(&b)[P], int st) __attribute__((always_inline)) {
#pragma unroll
      for (int q = 0; q < P; q++) {
        if constexpr (WP) b[q] = *(const u32x4_t *)(wrow + ((size_t)st * (HS / 4) + q) * wpstep);
        else b[q] = *(const u32x4_t *)(wrow + (size_t)st * HS * esz_w + 16 * q);
      }
    };
    auto wstep = [&](const u32x4_t(&b)[P], int st) __attribute__((always_inline)) {
      const int h = st * HS;
#pragma unroll
      for (int g = 0; g < HS / 8; g++) {
        float wf[8];
        if constexpr (WB) {
          const u32x4_t v = b[g];
          wf[0] = bf16_lo(v.x); wf[1] = bf16_hi(v.x); wf[2] = bf16_lo(v.y); wf[3] = bf16_hi(v.y);
          wf[4] = bf16_lo(v.z); wf[5] = bf16_hi(v.z); wf[6] = bf16_lo(v.w); wf[7] = bf16_hi(v.w);
        } else {
          const u32x4_t v0 = b[2 * g], v1 = b[2 * g + 1];
          wf[0] = __uint_as_float(v0.x); wf[1] = __uint_as_float(v0.y); wf[2] = __uint_as_float(v0.z);
          wf[3] = __uint_as_float(v0.w); wf[4] = __uint_as_float(v1.x); wf[5] = __uint_as_float(v1.y);
          wf[6] = __uint_as_float(v1.z); wf[7] = __uint_as_float(v1.w);
        }
#pragma unroll
        for (int tt = 0; tt < TT; tt++) {  // same LDS address in every lane: broadcast
          const f32x4_t xa = *(const f32x4_t *)(xs + tt * H + h + 8 * g);
          const f32x4_t xb = *(const f32x4_t *)(xs + tt * H + h + 8 * g + 4);
          const float xf[8] = {xa[0], xa[1], xa[2], xa[3], xb[0], xb[1], xb[2], xb[3]};
#pragma unroll
          for (int j = 0; j < 8; j++) acc[tt] = __builtin_fmaf(xf[j], wf[j], acc[tt]);
        }
      }
    };
    // The ring runs whole rounds with unconditional loads (steps past the end re-read the last
    // step, which is in bounds) and no exit inside a round, and a compiler barrier keeps every
    // load where it is issued: the number of loads issued after any slot is then fixed, so the
    // wait before a step covers only that step's slot.  A conditional load or an early exit makes
    // the compiler wait for every load in flight, and without the barrier it moves the loads next
    // to their use; either way a step then costs one memory round trip.
    if (nsteps > 0) {
#pragma unroll
      for (int q = 0; q < NS - 1; q++) wload(ring[q], q);
      asm volatile("" ::: "memory");
    }
    for (int st0 = 0; st0 < nsteps; st0 += NS) {
#pragma unroll
      for (int q = 0; q < NS; q++) {
        const int st = st0 + q;
        wload(ring[(q + NS - 1) % NS], min(st + NS - 1, nsteps - 1));
        asm volatile("" ::: "memory");
        wstep(ring[q], st);
      }
    }
    for (int h = nsteps * HS; h < H; h += 8) {
      float wf[8];
      if constexpr (WP) {
        const float4 a = *(const float4 *)(wrow + (size_t)(h / 4) * wpstep);
        const float4 b = *(const float4 *)(wrow + (size_t)(h / 4 + 1) * wpstep);
        wf[0] = a.x; wf[1] = a.y; wf[2] = a.z; wf[3] = a.w; wf[4] = b.x; wf[5] = b.y; wf[6] = b.z; wf[7] = b.w;
      } else {
        load8<WB>(wrow + (size_t)h * esz_w, wf);
      }
#pragma unroll
      for (int tt = 0; tt < TT; tt++) {
        const float *xp = xs + tt * H + h;
        const float xf[8] = {xp[0], xp[1], xp[2], xp[3], xp[4], xp[5], xp[6], xp[7]};
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
  asm volatile("" ::"v"(touch));  // keeps the warm-up loads
  if (active) {
#pragma unroll
    for (int tt = 0; tt < TT; tt++) lg[tt][e] = acc[tt];
  }
  __syncthreads();

  // top-k: wave c < EC handles tokens c, c+EC, ...
  for (int tt = c; active && tt < TT; tt += EC) {
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

// Top-k + gates of one token from its logits in LDS (wave-wide; every lane of the
// wave takes part).  Lanes own experts lane + 64q.
template <int EC>
__device__ __forceinline__ void topk_token(const float *lgt, int E, int k, int lane, int32_t *ids_t, float *gates_t) {
  uint64_t key[EC];
#pragma unroll
  for (int q = 0; q < EC; q++) {
    int eq = q * 64 + lane;
    key[q] = eq < E ? (((uint64_t)ord_key(lgt[eq]) << 32) | (uint32_t)~(uint32_t)eq) : 0ull;
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
    ids_t[lane] = my_e;
    gates_t[lane] = u / sum;
  }
}

}  // namespace rt

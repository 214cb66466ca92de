// Router GEMM + top-k + renormalised gates (moe_route).
//
// The router picks the top-K experts of every token (PagedAttention/MoE page,
// MoE list; AI-infra book, section 9.3.4).  The logit of (t, e) is an fp32
// fused-multiply-add chain over h in ascending order; this fixed order is the
// library's contract, so the chain is computed as is: one lane owns one expert
// and walks h upward; the token's activations are staged in LDS as fp32 and
// every lane reads them at one address (broadcast).  With few tokens the time
// is that of one wave issuing the chain (about 2.3 instructions per h), not
// memory.  Top-k is k rounds of a wave-wide max (DPP) over 64-bit
// keys (orderable logit bits, inverted expert id), so equal logits go to the
// lower expert index; the gates are a softmax over the k selected logits.
#include "permute_dev.h"

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
template <int TT, int EC, bool XB, bool WB, bool VEC, bool WP = false>
__device__ __forceinline__ void route_tokens(const void *__restrict__ x, const void *__restrict__ w,
                                             const float *__restrict__ bias, int T, int H, int E, int k,
                                             int32_t *__restrict__ ids, float *__restrict__ gates) {
  static_assert(!WP || (VEC && !WB), "the packed router weight is fp32, read 16 bytes at a time");
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
  const char *wrow = WP ? (const char *)w + (size_t)(ev ? e : 0) * 16 : (const char *)w + (size_t)(ev ? e : 0) * H * esz_w;
  const size_t wpstep = (size_t)E * 16;  // WP: bytes from one 4-wide h group to the next
  // Every block reads all of W_r, which is usually cold (the expert weights of the previous
  // layer call streamed through L2 since).  Each thread of the grid first touches one
  // distinct 128-byte line of it, so the whole matrix is pulled into L2 in one round trip
  // instead of block after block waiting on the same misses.
  uint32_t touch = 0;
  {
    const size_t nlines = (size_t)E * H * esz_w / 128;  // whole lines only: never past the end
    const size_t nthreads = (size_t)gridDim.x * blockDim.x;
    for (size_t l = (size_t)blockIdx.x * blockDim.x + threadIdx.x; l < nlines; l += nthreads)
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

  if constexpr (VEC) {
    // 32 h per step; a ring of ROUTE_NS register sets keeps the weight pieces of
    // the next ROUTE_NS-1 steps in flight while a step computes (each lane reads
    // its own expert row, so only prefetch depth hides the L2 latency)
    // fp32 weights take twice the registers per step: half the ring depth
    constexpr int HS = 32, P = HS * (WB ? 2 : 4) / 16, NS = WB ? ROUTE_NS : ROUTE_NS / 2;
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

template <int TT, int EC, bool XB, bool WB, bool VEC>
__global__ __launch_bounds__(64 * EC) void route_kernel(const void *__restrict__ x, const void *__restrict__ w,
                                                        const float *__restrict__ bias, int T, int H, int E, int k,
                                                        int32_t *__restrict__ ids, float *__restrict__ gates) {
  route_tokens<TT, EC, XB, WB, VEC>(x, w, bias, T, H, E, k, ids, gates);
}

// Decode route + local dispatch in one launch: block t routes token t (as route_kernel with one
// token per block) and zeroes row t of the fused-combine target; the last block to finish --
// found with a ticket counter, each block publishing its routing before it takes a ticket --
// groups the assignments by expert (the single-workgroup permutation) and resets the ticket.
// No block ever waits for another, so no co-residency is assumed.
template <int EC, bool XB, bool WB, bool WP>
__global__ __launch_bounds__(64 * EC) void route_dispatch_kernel(const void *__restrict__ x, const void *__restrict__ w,
                                                                 const float *__restrict__ bias, int T, int H, int E,
                                                                 int k, int lo, int El, int nbits,
                                                                 int32_t *__restrict__ ids, float *__restrict__ gates,
                                                                 int32_t *__restrict__ counts,
                                                                 int32_t *__restrict__ offsets,
                                                                 int32_t *__restrict__ row_token,
                                                                 float *__restrict__ row_w,
                                                                 int32_t *__restrict__ token_row,
                                                                 float *__restrict__ y_zero,
                                                                 uint32_t *__restrict__ ticket) {
  __shared__ int last;
  if (y_zero != nullptr) {
    f32x4_t *row = (f32x4_t *)(y_zero + (size_t)blockIdx.x * H);
    for (int i = threadIdx.x; i < H / 4; i += blockDim.x) row[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  route_tokens<1, EC, XB, WB, true, WP>(x, w, bias, T, H, E, k, ids, gates);
  __threadfence();  // this block's ids and gates are visible device-wide before its ticket
  __syncthreads();
  if (threadIdx.x == 0) last = atomicAdd(ticket, 1u) == (uint32_t)gridDim.x - 1u;
  __syncthreads();
  if (!last) return;
  __threadfence();  // acquire: every other block's routing
  extern __shared__ __attribute__((aligned(16))) float dyn[];
  const int N = T * k;
  const int R_cap = T * (k < El ? k : El);
  perm::permute_block<EC>(ids, gates, N, k, lo, El, nbits, R_cap, counts, offsets, row_token, row_w, token_row,
                          (int *)dyn);
  if (threadIdx.x == 0) atomicExch(ticket, 0u);
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

// Many tokens: the router weight and the workgroup's activations are staged
// through LDS in 64-wide h chunks, converted to fp32 once per workgroup (the
// next chunk is in registers while this one computes).  Every wave owns TR
// tokens, whose activations every lane reads at the same LDS address
// (broadcast), and every lane the experts lane + 64c.  The chain for each
// (token, expert) still runs h = 0, 1, 2, ... in order.  Needs H % 64 == 0.
template <int TR, int EC, bool XB, bool WB>
__global__ __launch_bounds__(256) void route_staged_kernel(const void *__restrict__ x, const void *__restrict__ w,
                                                           const float *__restrict__ bias, int T, int H, int E, int k,
                                                           int32_t *__restrict__ ids, float *__restrict__ gates) {
  constexpr int NW = 4, TB = NW * TR, HC = 64;
  constexpr int ROWS = 64 * EC;
  constexpr int LROW = HC + 4;                  // fp32 row stride in LDS (pad: conflict-free 16-byte reads)
  constexpr int WESZ = WB ? 2 : 4;
  constexpr int PIECES = ROWS * HC * WESZ / 16; // 16-byte global pieces per chunk
  constexpr int PPT = PIECES / 256;
  constexpr int PPR = HC * WESZ / 16;           // pieces per row
  __shared__ __attribute__((aligned(16))) float wl[ROWS * LROW];
  __shared__ __attribute__((aligned(16))) float xl[TB][LROW];  // this chunk of the block's activations, fp32
  __shared__ float lg[TB][ROWS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int XESZ = XB ? 2 : 4;
  constexpr int XPR = HC * XESZ / 16;   // 16-byte activation pieces per token row and chunk
  static_assert(TB * XPR <= 256, "one activation piece per thread");
  // activation piece of this thread (threads past TB*XPR have none)
  const bool xhas = tid < TB * XPR;
  const int xr = xhas ? tid / XPR : 0, xc = xhas ? tid % XPR : 0;
  const char *xsrc = (const char *)x + (size_t)min(blockIdx.x * TB + xr, T - 1) * H * XESZ + xc * 16;
  // staging pieces of this thread
  const char *src[PPT];
  int dst[PPT];
#pragma unroll
  for (int q = 0; q < PPT; q++) {
    const int pc = tid + 256 * q, row = pc / PPR, col = pc % PPR;
    const int er = row < E ? row : 0;
    src[q] = (const char *)w + ((size_t)er * H) * WESZ + col * 16;
    dst[q] = row * LROW + col * (16 / WESZ);
  }
  float acc[TR][EC];
#pragma unroll
  for (int t = 0; t < TR; t++)
#pragma unroll
    for (int c = 0; c < EC; c++) acc[t][c] = 0.0f;

  u32x4_t pre[PPT], xpre = {0, 0, 0, 0};
#pragma unroll
  for (int q = 0; q < PPT; q++) pre[q] = *(const u32x4_t *)src[q];
  if (xhas) xpre = *(const u32x4_t *)xsrc;
  for (int h0 = 0; h0 < H; h0 += HC) {
    // registers -> LDS as fp32
    if (xhas) {
      if constexpr (XB) {
        f32x4_t lo = {bf16_lo(xpre.x), bf16_hi(xpre.x), bf16_lo(xpre.y), bf16_hi(xpre.y)};
        f32x4_t hi = {bf16_lo(xpre.z), bf16_hi(xpre.z), bf16_lo(xpre.w), bf16_hi(xpre.w)};
        *(f32x4_t *)(&xl[xr][xc * 8]) = lo;
        *(f32x4_t *)(&xl[xr][xc * 8 + 4]) = hi;
      } else {
        *(u32x4_t *)(&xl[xr][xc * 4]) = xpre;
      }
    }
#pragma unroll
    for (int q = 0; q < PPT; q++) {
      if constexpr (WB) {
        const u32x4_t v = pre[q];
        f32x4_t lo = {bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y)};
        f32x4_t hi = {bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w)};
        *(f32x4_t *)(wl + dst[q]) = lo;
        *(f32x4_t *)(wl + dst[q] + 4) = hi;
      } else {
        *(u32x4_t *)(wl + dst[q]) = pre[q];
      }
    }
    __syncthreads();
    if (h0 + HC < H) {
#pragma unroll
      for (int q = 0; q < PPT; q++) pre[q] = *(const u32x4_t *)(src[q] + (size_t)(h0 + HC) * WESZ);
      if (xhas) xpre = *(const u32x4_t *)(xsrc + (size_t)(h0 + HC) * XESZ);
    }
#pragma unroll 2
    for (int hh = 0; hh < HC; hh += 8) {
      float xf[TR][8];
#pragma unroll
      for (int t = 0; t < TR; t++) {  // same address in every lane: broadcast reads
        const f32x4_t a = *(const f32x4_t *)(&xl[wave * TR + t][hh]), b = *(const f32x4_t *)(&xl[wave * TR + t][hh + 4]);
        xf[t][0] = a[0]; xf[t][1] = a[1]; xf[t][2] = a[2]; xf[t][3] = a[3];
        xf[t][4] = b[0]; xf[t][5] = b[1]; xf[t][6] = b[2]; xf[t][7] = b[3];
      }
#pragma unroll
      for (int c = 0; c < EC; c++) {
        const float *wr = wl + (lane + 64 * c) * LROW + hh;
        const f32x4_t w0 = *(const f32x4_t *)wr, w1 = *(const f32x4_t *)(wr + 4);
        const float wf[8] = {w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};
#pragma unroll
        for (int t = 0; t < TR; t++)
#pragma unroll
          for (int j = 0; j < 8; j++) acc[t][c] = __builtin_fmaf(xf[t][j], wf[j], acc[t][c]);
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int c = 0; c < EC; c++) {
    const int e = lane + 64 * c;
    const float b = (bias != nullptr && e < E) ? bias[e] : 0.0f;
#pragma unroll
    for (int t = 0; t < TR; t++) lg[wave * TR + t][e] = bias != nullptr ? acc[t][c] + b : acc[t][c];
  }
  __syncthreads();
  for (int tt = wave; tt < TB; tt += NW) {
    const int t = blockIdx.x * TB + tt;
    if (t >= T) break;
    topk_token<EC>(lg[tt], E, k, lane, ids + (size_t)t * k, gates + (size_t)t * k);
  }
}

template <int TT, int EC>
hipError_t launch_tt(const void *x, int xb, const void *w, int wb, const float *bias, int T, int H, int E, int k,
                     int32_t *ids, float *gates, hipStream_t s) {
  dim3 grid(ceil_div_i(T, TT)), block(64 * EC);
  const size_t xs_bytes = sizeof(float) * (size_t)TT * H;
  const bool vec = (H % 8 == 0) && (((uintptr_t)x | (uintptr_t)w) % 16 == 0) && xs_bytes <= 65536;
  const size_t shm = vec ? xs_bytes : 0;
#define ROUTE_CASE(XB, WB, V)                                                                                 \
  if (xb == XB && wb == WB && vec == V) {                                                                   \
    hipLaunchKernelGGL((route_kernel<TT, EC, XB, WB, V>), grid, block, shm, s, x, w, bias, T, H, E, k, ids, gates); \
    return hipGetLastError();                                                                               \
  }
  ROUTE_CASE(true, true, true) ROUTE_CASE(true, true, false) ROUTE_CASE(false, false, true)
  ROUTE_CASE(false, false, false) ROUTE_CASE(true, false, true) ROUTE_CASE(true, false, false)
  ROUTE_CASE(false, true, true) ROUTE_CASE(false, true, false)
#undef ROUTE_CASE
  return hipErrorInvalidValue;
}

// Tokens per wave of the staged kernel: 4 (16 per workgroup) while that still gives at least two
// workgroups per compute unit (512 on MI355X), else 3.  Measured on MI355X, moe_route alone:
// T = 6000: 3 -> 166 us, 4 -> 186 us (375 workgroups); T = 8192: 3 -> 218 us, 4 -> 196 us.
template <int TR, int EC>
hipError_t launch_staged_tr(const void *x, int xb, const void *w, int wb, const float *bias, int T, int H, int E,
                            int k, int32_t *ids, float *gates, hipStream_t s) {
  constexpr int TB = 4 * TR;
  dim3 grid(ceil_div_i(T, TB)), block(256);
#define STAGED_CASE(XB, WB)                                                                                      \
  if (xb == XB && wb == WB) {                                                                                  \
    hipLaunchKernelGGL((route_staged_kernel<TR, EC, XB, WB>), grid, block, 0, s, x, w, bias, T, H, E, k, ids, gates); \
    return hipGetLastError();                                                                                  \
  }
  STAGED_CASE(true, true) STAGED_CASE(false, false) STAGED_CASE(true, false) STAGED_CASE(false, true)
#undef STAGED_CASE
  return hipErrorInvalidValue;
}

template <int EC>
hipError_t launch_staged(const void *x, int xb, const void *w, int wb, const float *bias, int T, int H, int E, int k,
                         int32_t *ids, float *gates, hipStream_t s) {
  if (ceil_div_i(T, 16) >= 512) return launch_staged_tr<4, EC>(x, xb, w, wb, bias, T, H, E, k, ids, gates, s);
  return launch_staged_tr<3, EC>(x, xb, w, wb, bias, T, H, E, k, ids, gates, s);
}

template <int EC>
hipError_t launch_ec(const void *x, int xb, const void *w, int wb, const float *bias, int T, int H, int E, int k,
                     int32_t *ids, float *gates, hipStream_t s) {
  // Few tokens: one token per block keeps every chain on its own wave (latency).
  // Many tokens: the LDS-staged kernel shares each weight chunk among 4*TR tokens.
  const bool aligned = (((uintptr_t)x | (uintptr_t)w) % 16 == 0);
  if constexpr (EC <= 2) {
    if (T > 256 && H % 64 == 0 && aligned) return launch_staged<EC>(x, xb, w, wb, bias, T, H, E, k, ids, gates, s);
  }
  if (T <= 512) return launch_tt<1, EC>(x, xb, w, wb, bias, T, H, E, k, ids, gates, s);
  return launch_tt<4, EC>(x, xb, w, wb, bias, T, H, E, k, ids, gates, s);
}

}  // namespace

namespace {

template <int EC>
hipError_t launch_rd(const void *x, int xb, const void *w, int wb, const float *bias, int T, int H, int E, int k, int lo,
                     int El, int32_t *ids, float *gates, int32_t *counts, int32_t *offsets, int32_t *row_token,
                     float *row_w, int32_t *token_row, float *y_zero, uint32_t *ticket, hipStream_t s) {
  int nbits = 0;
  while ((1 << nbits) < El) nbits++;
  const size_t xs_bytes = sizeof(float) * (size_t)H, perm_bytes = sizeof(int) * (size_t)(EC + 1) * El;
  const size_t shm = xs_bytes > perm_bytes ? xs_bytes : perm_bytes;
  // wb: 0 fp32 row-major, 1 bf16 row-major, 2 fp32 in the layout of moe_pack_router
#define RD_CASE(XB, WB, WP)                                                                                      \
  if (xb == XB && wb == (WP ? 2 : (WB ? 1 : 0))) {                                                               \
    hipLaunchKernelGGL((route_dispatch_kernel<EC, XB, WB, WP>), dim3(T), dim3(64 * EC), shm, s, x, w, bias, T, H, E, \
                       k, lo, El, nbits, ids, gates, counts, offsets, row_token, row_w, token_row, y_zero, ticket); \
    return hipGetLastError();                                                                                    \
  }
  RD_CASE(true, true, false) RD_CASE(false, false, false) RD_CASE(true, false, false) RD_CASE(false, true, false)
  RD_CASE(true, false, true) RD_CASE(false, false, true)
#undef RD_CASE
  return hipErrorInvalidValue;
}

}  // namespace

bool route_dispatch_fits(int T, int H, int E, int k, const void *x, const void *w) {
  return T >= 1 && T <= kRouteDispatchMaxT && (long long)T * k <= 8192 && E <= 256 && H % 8 == 0 &&
         H * sizeof(float) <= 65536 && (((uintptr_t)x | (uintptr_t)w) % 16 == 0);
}

hipError_t launch_route_dispatch(const void *x, int x_bf16, const void *w, int w_bf16, const float *bias, int T, int H,
                                 int E, int k, int lo, int El, int32_t *ids, float *gates, int32_t *counts,
                                 int32_t *offsets, int32_t *row_token, float *row_w, int32_t *token_row,
                                 float *y_zero, uint32_t *ticket, hipStream_t s) {
  if (E <= 64)
    return launch_rd<1>(x, x_bf16, w, w_bf16, bias, T, H, E, k, lo, El, ids, gates, counts, offsets, row_token, row_w,
                        token_row, y_zero, ticket, s);
  if (E <= 128)
    return launch_rd<2>(x, x_bf16, w, w_bf16, bias, T, H, E, k, lo, El, ids, gates, counts, offsets, row_token, row_w,
                        token_row, y_zero, ticket, s);
  return launch_rd<4>(x, x_bf16, w, w_bf16, bias, T, H, E, k, lo, El, ids, gates, counts, offsets, row_token, row_w,
                      token_row, y_zero, ticket, s);
}

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

namespace {
// [E, H] (bf16 or fp32) -> [H/4][E][4] fp32: out[(j E + e) 4 + i] = w[e, 4j + i] (exact for bf16).
__global__ __launch_bounds__(256) void pack_router_kernel(const void *__restrict__ w, int wbf16, int E, int H,
                                                          float *__restrict__ out) {
  const size_t n = (size_t)E * (H / 4);
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
    const size_t j = i / E, e = i - j * E;  // output piece i = j E + e
    const size_t src = e * (size_t)H + 4 * j;
    f32x4_t v;
    if (wbf16) {
      const uint16_t *b = (const uint16_t *)w + src;
      v = f32x4_t{bf16_to_f32(b[0]), bf16_to_f32(b[1]), bf16_to_f32(b[2]), bf16_to_f32(b[3])};
    } else {
      const float *f = (const float *)w + src;
      v = f32x4_t{f[0], f[1], f[2], f[3]};
    }
    *(f32x4_t *)(out + 4 * i) = v;
  }
}
}  // namespace

hipError_t launch_pack_router(const void *w, int w_bf16, int E, int H, float *out, hipStream_t s) {
  const size_t n = (size_t)E * (H / 4);
  if (n == 0) return hipSuccess;
  const size_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(pack_router_kernel, dim3(blocks < 4096 ? (unsigned)blocks : 4096u), dim3(256), 0, s, w, w_bf16,
                     E, H, out);
  return hipGetLastError();
}

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
#include "route_dev.h"

namespace {

using namespace rt;

// Up to 1024 experts: 16 waves per block (four per SIMD) leave 128 registers per lane, so the weight
// ring is half as deep there.
template <int TT, int EC, bool XB, bool WB, bool VEC>
__global__ __launch_bounds__(64 * EC) void route_kernel(const void *__restrict__ x, const void *__restrict__ w,
                                                        const float *__restrict__ bias, int T, int H, int E, int k,
                                                        int32_t *__restrict__ ids, float *__restrict__ gates) {
  constexpr int ring = EC >= 16 ? ROUTE_NS / 2 : ROUTE_NS;
  route_tokens<TT, EC, XB, WB, VEC, false, ring>(x, w, bias, T, H, E, k, ids, gates, blockIdx.x * TT, blockIdx.x,
                                                 gridDim.x);
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
  route_tokens<1, EC, XB, WB, true, WP>(x, w, bias, T, H, E, k, ids, gates, blockIdx.x, blockIdx.x, gridDim.x);
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
    case 5:
    case 6:
    case 7:
    case 8: return launch_ec<8>(x, x_bf16, w, w_bf16, bias, T, H, E, k, ids, gates, s);
    default: return launch_ec<16>(x, x_bf16, w, w_bf16, bias, T, H, E, k, ids, gates, s);
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

// The whole MoE layer of a decode batch in one persistent launch (moe_decode_layer).
//
// "Hosting Qwen on Blackwell", section "Expert parallelism": for decoding the whole MoE kernel is
// merged into one.  Here one launch runs routing (router GEMM, top-k, gates), the grouping of the
// assignments by expert, the SwiGLU gate/up projection, and the down projection with the gate-
// weighted combine into y, and the weight stream of the expert GEMMs starts at once instead of
// after the router, whose 4096-long fp32 chains are latency bound and leave HBM idle.
//
// Work items, claimed in order from one atomic queue by the resident workgroups:
//   [0, T)                    route token t; the last routing item to finish (ticket counter)
//                             groups all assignments by expert and raises the ``routed`` flag;
//   [T, T + El*NBg)           gate/up item (expert e, 128 intermediate columns), h into a dense
//                             [El, T, I] buffer (row = token), after the flag: only the expert's
//                             rows, and nothing for an expert without rows.  (Starting these items
//                             before the routing is known, over every token of the batch so that
//                             the weights stream while the router runs, measured slower: the
//                             router's dependent loads slow down once they compete with the weight
//                             stream, and every wave then reads twice the activations);
//   [.., + El*NBd)            down item (expert e, 256 output columns) over the expert's rows, whose
//                             h rows it gathers by token, after the flag and the NBg gate/up items
//                             of e (per-expert completion counter).
// Each h value is the same MFMA sequence as in the weight-streaming grouped kernel, so the rows
// the routing selects are bit-identical to moe_grouped_ffn's.
//
// Every wait is for items claimed earlier, i.e. owned by workgroups that are already running and
// that only wait for still earlier items, so the waits always end; the grid is also no larger than
// the number of workgroups the device holds at once.  Each wait is bounded all the same: past
// kSpinLimit polls it sets an error bit in the workspace and the item gives up.
//
// Cross-workgroup data (routing results, h) crosses the per-XCD L2 caches with agent-scope
// release fences (write-back) before the counters and flags, and agent-scope loads or one
// acquire fence (invalidate) after them.  The last workgroup to leave resets the control words,
// so every call leaves them zero.
#include "ffn_common.h"
#include "permute_dev.h"
#include "route_dev.h"
#include "stream_core.h"

#include <mutex>

namespace {

constexpr int NWAVE = 4, NTHR = 64 * NWAVE;
constexpr int SMB = 2, MT = 32 * SMB;  // 64-row M tiles (two 32-row MFMA blocks)
constexpr int GU_COLS = 32 * NWAVE;    // intermediate columns of a gate/up item (32 per wave)
constexpr int DN_COLS = 64 * NWAVE;    // output columns of a down item (64 per wave)
constexpr uint32_t kSpinLimit = 1u << 20;


struct DecParams {
  const void *x;            // [T, H] bf16
  const void *wr;           // router weight: [E, H] bf16 / fp32, or [H/4, E, 4] fp32 (moe_pack_router)
  const float *bias;        // [E] or NULL
  int T, H, E, k, lo, El, nbits, R_cap, I;
  int32_t *ids;             // [T, k]
  float *gates;             // [T, k]
  int32_t *counts, *offsets, *row_token, *token_row;
  float *row_w;
  float *y;                 // [T, H] fp32, zeroed by the routing items, then accumulated
  const void *wgu, *wd;     // [El, 2I, H], [El, H, I] (bf16 or e4m3; row-major or packed)
  const float *sgu, *sd;    // e4m3 per-channel scales [El, 2I], [El, H]
  int wpacked;
  uint16_t *h;              // [El, T, I] bf16 (dense: every token of every local expert)
  uint32_t *ctl;            // control words (DecCtl), zero before the call
  int n_gu, n_items, NBg, NBd;
};

// The item functions are not inlined into the kernel (see decode_layer_kernel), so the compiler no
// longer knows that the pointers in DecParams address global memory and would use flat (generic)
// memory instructions.  Each item function therefore starts from a copy of the parameters whose
// pointers went through the global address space (the casts cost nothing; loads, stores and atomics
// through them become global_* instructions).
template <typename T>
__device__ __forceinline__ T *glob(T *q) {
  return (T *)(__attribute__((address_space(1))) T *)q;
}

__device__ __forceinline__ DecParams global_params(const DecParams &in) {
  DecParams p = in;
  p.x = glob(p.x);
  p.wr = glob(p.wr);
  p.bias = glob(p.bias);
  p.ids = glob(p.ids);
  p.gates = glob(p.gates);
  p.counts = glob(p.counts);
  p.offsets = glob(p.offsets);
  p.row_token = glob(p.row_token);
  p.token_row = glob(p.token_row);
  p.row_w = glob(p.row_w);
  p.y = glob(p.y);
  p.wgu = glob(p.wgu);
  p.wd = glob(p.wd);
  p.sgu = glob(p.sgu);
  p.sd = glob(p.sd);
  p.h = glob(p.h);
  p.ctl = glob(p.ctl);
  return p;
}

__device__ __forceinline__ uint32_t ld_agent(const uint32_t *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t ld_agent(const int32_t *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One thread: wait until *w >= v; gives up (error bit ``code``) after kSpinLimit polls.  With
// ``acquire`` an acquire fence follows (this CU's L1 and this XCD's L2 are invalidated, so plain
// loads see what other workgroups released); without it only agent-scope loads (which bypass the
// non-coherent caching) may read the data the counter guards -- that keeps the activations cached
// in L2 for the gate/up items that share this XCD.
__device__ __forceinline__ bool wait_at_least(const DecParams &p, uint32_t *w, uint32_t v, uint32_t code, bool acquire) {
  for (uint32_t i = 0; i < kSpinLimit; i++) {
    if (ld_agent(w) >= v) {
      if (acquire) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      return true;
    }
    __builtin_amdgcn_s_sleep(2);
  }
  atomicOr(p.ctl + kDecError, code);
  return false;
}

// Route token t: zero its row of y, its logits / top-k / gates, then the ticket; the last routing
// item groups the assignments (the single-workgroup permutation) and raises the flag.
template <int EC, bool WB, bool WP>
__device__ __noinline__ void route_item(const DecParams &pin, int t, int *smem) {
  const DecParams p = global_params(pin);
  f32x4_t *yrow = (f32x4_t *)(p.y + (size_t)t * p.H);
  for (int i = threadIdx.x; i < p.H / 4; i += NTHR) yrow[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  rt::route_tokens<1, EC, true, WB, true, WP>(p.x, p.wr, p.bias, p.T, p.H, p.E, p.k, p.ids, p.gates, t, t, p.T);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");  // y row, ids and gates before the ticket
  __syncthreads();
  __shared__ int last;
  if (threadIdx.x == 0) last = atomicAdd(p.ctl + kDecTicket, 1u) == (uint32_t)p.T - 1u;
  __syncthreads();
  if (!last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // every routing item's ids and gates
  perm::permute_block<NWAVE>(p.ids, p.gates, p.T * p.k, p.k, p.lo, p.El, p.nbits, p.R_cap, p.counts, p.offsets,
                             p.row_token, p.row_w, p.token_row, smem);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_store(p.ctl + kDecRouted, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

// This lane's first weight piece of row ``row`` (counted over all experts) at k = 0, k offset 32g.
template <bool FP8>
__device__ __forceinline__ const char *weight_lane(const DecParams &p, const void *w, size_t row, int K, int g) {
  constexpr int wesz = FP8 ? 1 : 2;
  return (const char *)w + ffn::w_piece_off(p.wpacked, row, 2 * wesz * g, K, wesz);
}

template <bool FP8>
__device__ __noinline__ void gate_up_item(const DecParams &pin, int e, int nb, int *s) {
  const DecParams p = global_params(pin);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, n = lane & 31, g = lane >> 5;
  if (threadIdx.x == 0) {  // the grouping (agent-scope loads only); a wait that gives up leaves no rows
    const bool routed = wait_at_least(p, p.ctl + kDecRouted, 1u, 16u, false);
    const int beg = routed ? ld_agent(p.offsets + e) : 0;
    s[1] = beg;
    s[2] = routed ? ld_agent(p.offsets + e + 1) - beg : 0;
  }
  __syncthreads();
  // wave-uniform (the same LDS words in every lane)
  const int beg = __builtin_amdgcn_readfirstlane(s[1]), rows = __builtin_amdgcn_readfirstlane(s[2]);
  const int c0 = nb * GU_COLS + wave * 32;
  // only the expert's rows (none: skip, no weight read)
  if (rows > 0 && c0 < p.I) {  // I is a multiple of 32: a wave's columns are all valid or all past the end
    const int col = c0 + n;
    const char *wrow[2] = {weight_lane<FP8>(p, p.wgu, (size_t)e * 2 * p.I + col, p.H, g),
                           weight_lane<FP8>(p, p.wgu, (size_t)e * 2 * p.I + p.I + col, p.H, g)};
    float sg = 1.0f, su = 1.0f;
    if constexpr (FP8) {
      sg = p.sgu[(size_t)e * 2 * p.I + col];
      su = p.sgu[(size_t)e * 2 * p.I + p.I + col];
    }
    // token of tile row m (rows past the end repeat the last one)
    auto token = [&](int m) { return ld_agent(p.row_token + beg + min(m, rows - 1)); };
    const uint16_t *arow[SMB];
#pragma unroll
    for (int mb = 0; mb < SMB; mb++) arow[mb] = (const uint16_t *)p.x + (size_t)token(mb * 32 + n) * p.H + 32 * g;
    f32x16_t acc[SMB][2];
    sc::zero_acc(acc);
    sc::stream_mfma<FP8, SMB, 2>(wrow, ffn::w_lane_piece_step(p.wpacked, FP8 ? 1 : 2),
                                 ffn::w_chunk_step(p.wpacked, FP8 ? 1 : 2), arow, rows > 32, p.H / 64, acc);
    uint16_t *hcol = p.h + (size_t)e * p.T * p.I + col;
#pragma unroll
    for (int mb = 0; mb < SMB; mb++) {
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int m = mb * 32 + sc::acc_row(r, lane);
        if (m < rows)
          hcol[(size_t)token(m) * p.I] = f32_to_bf16(silu_fast(acc[mb][0][r] * sg) * (acc[mb][1][r] * su));
      }
    }
  }
  // every wave's h stores have reached the L2; then one write-back of this XCD's L2 and the count
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __hip_atomic_fetch_add(p.ctl + kDecDone + e, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <bool FP8>
__device__ __noinline__ void down_item(const DecParams &pin, int e, int nb, int *s) {
  const DecParams p = global_params(pin);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, n = lane & 31, g = lane >> 5;
  if (threadIdx.x == 0) {
    bool ok = wait_at_least(p, p.ctl + kDecRouted, 1u, 4u, false);
    int beg = 0, cnt = 0;
    if (ok) {
      beg = ld_agent(p.offsets + e);
      cnt = ld_agent(p.offsets + e + 1) - beg;
    }
    // the expert's h rows are complete; the acquire makes them (and the grouping, released before
    // the flag every gate/up item saw) visible to plain loads
    if (cnt > 0 && !wait_at_least(p, p.ctl + kDecDone + e, (uint32_t)p.NBg, 8u, true)) cnt = 0;
    s[1] = beg;
    s[2] = cnt;
  }
  __syncthreads();
  const int beg = __builtin_amdgcn_readfirstlane(s[1]), cnt = __builtin_amdgcn_readfirstlane(s[2]);
  if (cnt == 0) return;
  const int c0 = nb * DN_COLS + wave * 64;
  const bool on = c0 < p.H;  // wave-uniform: H is a multiple of 64
  const int cw = on ? c0 : p.H - 64;
  const int col = cw + n;
  const char *wrow[2] = {weight_lane<FP8>(p, p.wd, (size_t)e * p.H + col, p.I, g),
                         weight_lane<FP8>(p, p.wd, (size_t)e * p.H + col + 32, p.I, g)};
  const size_t cstep = ffn::w_chunk_step(p.wpacked, FP8 ? 1 : 2);
  float sd[2] = {1.0f, 1.0f};
  if constexpr (FP8) {
    sd[0] = p.sd[(size_t)e * p.H + col];
    sd[1] = p.sd[(size_t)e * p.H + col + 32];
  }
  if (!on) return;
  for (int m0 = 0; m0 < cnt; m0 += MT) {
    const int rows = min(MT, cnt - m0), r0 = beg + m0;
    const uint16_t *arow[SMB];
#pragma unroll
    for (int mb = 0; mb < SMB; mb++)
      arow[mb] = p.h + ((size_t)e * p.T + p.row_token[r0 + min(mb * 32 + n, rows - 1)]) * p.I + 32 * g;
    f32x16_t acc[SMB][2];
    sc::zero_acc(acc);
    sc::stream_mfma<FP8, SMB, 2>(wrow, ffn::w_lane_piece_step(p.wpacked, FP8 ? 1 : 2), cstep, arow, rows > 32,
                                 p.I / 64, acc);
#pragma unroll
    for (int b = 0; b < 2; b++) {
#pragma unroll
      for (int mb = 0; mb < SMB; mb++) {
#pragma unroll
        for (int r = 0; r < 16; r++) {
          const int m = mb * 32 + sc::acc_row(r, lane);
          if (m < rows) {
            const int row = r0 + m;
            atomicAdd(p.y + (size_t)p.row_token[row] * p.H + col + 32 * b, p.row_w[row] * (acc[mb][b][r] * sd[b]));
          }
        }
      }
    }
  }
}

// The three item kinds are separate (not inlined) functions: each gets its own register allocation,
// within the two-waves-per-SIMD budget, instead of the union of all three.
template <int EC, bool WB, bool WP, bool FP8>
__global__ __launch_bounds__(NTHR, 2) void decode_layer_kernel(DecParams p) {  // two waves per SIMD
  extern __shared__ __attribute__((aligned(16))) int dsm[];  // x staging of the router / permutation scratch
  __shared__ int s_item;
  __shared__ int s_tile[4];
  for (;;) {
    if (threadIdx.x == 0) s_item = (int)atomicAdd(p.ctl + kDecQueue, 1u);
    __syncthreads();
    const int item = __builtin_amdgcn_readfirstlane(s_item);
    __syncthreads();  // everyone has the item before thread 0 may claim the next one
    if (item >= p.n_items) break;
    if (item < p.T) {
      route_item<EC, WB, WP>(p, item, dsm);
    } else if (item < p.T + p.n_gu) {
      const int j = item - p.T;
      gate_up_item<FP8>(p, j / p.NBg, j % p.NBg, s_tile);
    } else {
      const int j = item - p.T - p.n_gu;
      down_item<FP8>(p, j / p.NBd, j % p.NBd, s_tile);
    }
    __syncthreads();
  }
  if (threadIdx.x == 0 && atomicAdd(p.ctl + kDecExit, 1u) == gridDim.x - 1u) {
    // every other workgroup has left: zero the control words for the next call (not the error word)
    for (int i = 0; i < kDecError; i++) __hip_atomic_store(p.ctl + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int e = 0; e < p.El; e++)
      __hip_atomic_store(p.ctl + kDecDone + e, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Workgroups the device holds at once, per device and kernel instance (queried once).
template <typename K>
int resident_blocks(K kernel, size_t shm) {
  static std::mutex mu;
  static int cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  std::lock_guard<std::mutex> lock(mu);
  if (cache[dev] == 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, NTHR, shm) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    cache[dev] = per_cu * cus;
  }
  return cache[dev];
}

template <int EC, bool WB, bool WP, bool FP8>
hipError_t launch_k(const DecParams &p, size_t shm, hipStream_t s) {
  auto kernel = decode_layer_kernel<EC, WB, WP, FP8>;
  const int resident = resident_blocks(kernel, shm);
  if (resident <= 0) return hipErrorInvalidConfiguration;
  const int grid = p.n_items < resident ? p.n_items : resident;
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(NTHR), shm, s, p);
  return hipGetLastError();
}

template <int EC>
hipError_t launch_ec(const DecParams &p, int wmode, bool fp8, size_t shm, hipStream_t s) {
  // wmode: 0 fp32 row-major router weight, 1 bf16 row-major, 2 fp32 packed (moe_pack_router)
  if (wmode == 1) return fp8 ? launch_k<EC, true, false, true>(p, shm, s) : launch_k<EC, true, false, false>(p, shm, s);
  if (wmode == 2) return fp8 ? launch_k<EC, false, true, true>(p, shm, s) : launch_k<EC, false, true, false>(p, shm, s);
  return fp8 ? launch_k<EC, false, false, true>(p, shm, s) : launch_k<EC, false, false, false>(p, shm, s);
}

}  // namespace

size_t decode_layer_ws_bytes(int T, int k, int El, int I) {
  (void)k;
  return align_up((size_t)(kDecDone + El) * 4, 256) + align_up((size_t)El * T * (size_t)I * 2, 256);
}

hipError_t launch_decode_layer(const DecodeArgs &a, hipStream_t s) {
  DecParams p{};
  p.x = a.x;
  p.wr = a.wr;
  p.bias = a.bias;
  p.T = a.T;
  p.H = a.H;
  p.E = a.E;
  p.k = a.k;
  p.lo = a.lo;
  p.El = a.El;
  int nbits = 0;
  while ((1 << nbits) < a.El) nbits++;
  p.nbits = nbits;
  p.R_cap = a.T * (a.k < a.El ? a.k : a.El);
  p.I = a.I;
  p.ids = a.ids;
  p.gates = a.gates;
  p.counts = a.counts;
  p.offsets = a.offsets;
  p.row_token = a.row_token;
  p.row_w = a.row_w;
  p.token_row = a.token_row;
  p.y = a.y;
  p.wgu = a.wgu;
  p.wd = a.wd;
  p.sgu = a.sgu;
  p.sd = a.sd;
  p.wpacked = a.wpacked;
  p.ctl = (uint32_t *)a.ws;
  p.h = (uint16_t *)((char *)a.ws + align_up((size_t)(kDecDone + a.El) * 4, 256));
  p.NBg = ceil_div_i(a.I, GU_COLS);
  p.NBd = ceil_div_i(a.H, DN_COLS);
  p.n_gu = a.El * p.NBg;
  p.n_items = a.T + p.n_gu + a.El * p.NBd;
  const size_t xs = sizeof(float) * (size_t)a.H, perm = sizeof(int) * (size_t)(NWAVE + 1) * a.El;
  const size_t shm = xs > perm ? xs : perm;
  const int ec = ceil_div_i(a.E, 64);
  if (ec == 1) return launch_ec<1>(p, a.wmode, a.fp8, shm, s);
  if (ec == 2) return launch_ec<2>(p, a.wmode, a.fp8, shm, s);
  return launch_ec<4>(p, a.wmode, a.fp8, shm, s);
}

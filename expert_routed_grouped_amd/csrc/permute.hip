// Local dispatch (moe_permute): per-expert counts, offsets and the stable
// grouping of assignments by expert, plus the optional row gather x -> x_perm.
//
// Dispatch groups every expert's tokens into the GEMM input buffers and, with
// replicated inputs, keeps only the tokens of the local experts ("Hosting Qwen
// on Blackwell", sections "MoE Dispatch - Combine" and "Expert parallelism");
// the per-expert row counts m_j are the AI-infra book's load measure (section
// 9.4.2) and the padding unit of the grouped GEMM (section 9.4.3).
//
// One workgroup of 16 waves does the whole (small) integer problem without any
// host synchronisation: each wave owns a contiguous slice of the assignments in
// token-major order.  Pass 1 counts, per wave and expert, with a wave-wide
// "match" (lanes holding the same expert found with one ballot per expert-id
// bit) so only one lane per expert touches LDS.  A scan over experts and waves
// then gives every wave its starting row inside every expert.  Pass 2 repeats
// the match and hands out rows by lane rank, which keeps the rows of one expert
// in increasing token order: the unique stable order.
#include "common.h"

namespace {

constexpr int kPermWaves = 16;
constexpr int kPermThreads = kPermWaves * 64;
constexpr int kUnroll = 8;  // loads in flight per lane before the batch is processed

__device__ __forceinline__ uint64_t lanemask_lt(int lane) { return (lane == 0) ? 0ull : (~0ull >> (64 - lane)); }

// Lanes whose ``key`` equals this lane's key, among lanes with ``active`` set.
__device__ __forceinline__ uint64_t match_lanes(int key, bool active, int nbits) {
  uint64_t m = __ballot(active);
  for (int b = 0; b < nbits; b++) {
    bool bit = (key >> b) & 1;
    uint64_t ones = __ballot(active && bit);
    m &= bit ? ones : ~ones;
  }
  return m;
}

__global__ __launch_bounds__(kPermThreads) void permute_kernel(const int32_t *__restrict__ ids,
                                                              const float *__restrict__ w, int N, int k, int lo,
                                                              int El, int nbits, int R_cap,
                                                              int32_t *__restrict__ counts,
                                                              int32_t *__restrict__ offsets,
                                                              int32_t *__restrict__ row_token,
                                                              float *__restrict__ row_w,
                                                              int32_t *__restrict__ token_row) {
  extern __shared__ int smem[];
  int *cnt = smem;                  // [kPermWaves][El]: per-wave counts, then per-wave next row
  int *scan = smem + kPermWaves * El;  // [El]
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < kPermWaves * El; i += kPermThreads) cnt[i] = 0;
  __syncthreads();

  const int per = ((N + kPermThreads - 1) / kPermThreads) * 64;  // multiple of 64
  const int a0 = min(N, wave * per), a1 = min(N, a0 + per);

  // ---- pass 1: per-wave, per-expert counts
  for (int base = a0; base < a1; base += 64 * kUnroll) {
    int ev[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; u++) {
      int a = base + u * 64 + lane;
      ev[u] = a < a1 ? ids[a] - lo : -1;
    }
#pragma unroll
    for (int u = 0; u < kUnroll; u++) {
      if (base + u * 64 >= a1) break;
      bool local = (unsigned)ev[u] < (unsigned)El;
      uint64_t peers = match_lanes(ev[u], local, nbits);
      if (local && (peers & lanemask_lt(lane)) == 0) cnt[wave * El + ev[u]] += __popcll(peers);
    }
  }
  __syncthreads();

  // ---- scan: offsets over experts, then each wave's first row in each expert
  for (int e = threadIdx.x; e < El; e += kPermThreads) {
    int s = 0;
    for (int v = 0; v < kPermWaves; v++) s += cnt[v * El + e];
    scan[e] = s;
    counts[e] = s;
  }
  __syncthreads();
  if (wave == 0) {
    // exclusive scan of scan[0..El) by one wave, 64 experts at a time
    int carry = 0;
    for (int b = 0; b < El; b += 64) {
      int e = b + lane;
      int v = e < El ? scan[e] : 0;
      int incl = v;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        int o = __shfl_up(incl, off, 64);
        if (lane >= off) incl += o;
      }
      if (e < El) scan[e] = carry + incl - v;
      carry += __shfl(incl, 63, 64);
    }
    if (lane == 0) offsets[El] = carry;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < El; e += kPermThreads) {
    int run = scan[e];
    offsets[e] = run;
    for (int v = 0; v < kPermWaves; v++) {
      int c = cnt[v * El + e];
      cnt[v * El + e] = run;
      run += c;
    }
  }
  __syncthreads();

  // ---- pass 2: rows
  for (int base = a0; base < a1; base += 64 * kUnroll) {
    int ev[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; u++) {
      int a = base + u * 64 + lane;
      ev[u] = a < a1 ? ids[a] - lo : -1;
    }
#pragma unroll
    for (int u = 0; u < kUnroll; u++) {
      const int a = base + u * 64 + lane;
      if (base + u * 64 >= a1) break;
      const bool valid = a < a1;
      const bool local = (unsigned)ev[u] < (unsigned)El;
      uint64_t peers = match_lanes(ev[u], local, nbits);
      int rank = __popcll(peers & lanemask_lt(lane));
      int r = -1;
      if (local) {
        int slot = wave * El + ev[u];
        int first = cnt[slot];
        r = first + rank;
        if (rank == 0) cnt[slot] = first + __popcll(peers);
        if (r < R_cap) {  // always true for distinct experts per token; guards bad input
          row_token[r] = a / k;
          row_w[r] = w[a];
        }
      }
      if (valid) token_row[a] = r < R_cap ? r : -1;
    }
  }
}

// x_perm[r] = x[row_token[r]] for r < offsets[El]; 16-byte vectors.
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint4 *__restrict__ x, int row_vecs,
                                                          const int32_t *__restrict__ offsets, int El,
                                                          const int32_t *__restrict__ row_token, int R_cap,
                                                          uint4 *__restrict__ x_perm) {
  const int R = min(offsets[El], R_cap);
  for (int r = blockIdx.x; r < R; r += gridDim.x) {
    const uint4 *src = x + (size_t)row_token[r] * row_vecs;
    uint4 *dst = x_perm + (size_t)r * row_vecs;
    for (int i = threadIdx.x; i < row_vecs; i += blockDim.x) dst[i] = src[i];
  }
}

}  // namespace

hipError_t launch_permute(const int32_t *ids, const float *w, int T, int k, int lo, int El, int32_t *counts,
                          int32_t *offsets, int32_t *row_token, float *row_w, int32_t *token_row, hipStream_t s) {
  int nbits = 0;
  while ((1 << nbits) < El) nbits++;
  size_t shm = sizeof(int) * (size_t)(kPermWaves + 1) * El;
  const int R_cap = T * (k < El ? k : El);
  hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(kPermThreads), shm, s, ids, w, T * k, k, lo, El, nbits, R_cap,
                     counts, offsets, row_token, row_w, token_row);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const void *x, int esz, int H, const int32_t *offsets, int El, const int32_t *row_token,
                              int R_cap, void *x_perm, hipStream_t s) {
  if (R_cap == 0) return hipSuccess;
  int row_vecs = H * esz / 16;
  int grid = R_cap < 4096 ? R_cap : 4096;
  hipLaunchKernelGGL(gather_rows_kernel, dim3(grid), dim3(256), 0, s, (const uint4 *)x, row_vecs, offsets, El,
                     row_token, R_cap, (uint4 *)x_perm);
  return hipGetLastError();
}

// Stable grouping of assignments by expert, shared by the permutation kernels
// (permute.hip) and the fused decode route + dispatch kernel (route.hip).
#pragma once
#include "common.h"

namespace perm {

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

// Count, per expert, the local assignments a in [a0, a1) of one wave into cnt[] (LDS).
__device__ __forceinline__ void wave_count(const int32_t *__restrict__ ids, int a0, int a1, int lo, int El, int nbits,
                                           int *cnt, int lane) {
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
      if (local && (peers & lanemask_lt(lane)) == 0) cnt[ev[u]] += __popcll(peers);
    }
  }
}

// Give rows to the assignments a in [a0, a1) of one wave, in order; next[e] (LDS)
// holds this wave's next free row of expert e and is advanced.
__device__ __forceinline__ void wave_assign(const int32_t *__restrict__ ids, const float *__restrict__ w, int a0,
                                            int a1, int k, int lo, int El, int nbits, int R_cap, int *next, int lane,
                                            int32_t *__restrict__ row_token, float *__restrict__ row_w,
                                            int32_t *__restrict__ token_row) {
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
        int first = next[ev[u]];
        r = first + rank;
        if (rank == 0) next[ev[u]] = first + __popcll(peers);
        if (r < R_cap) {  // always true for distinct experts per token; guards bad input
          row_token[r] = a / k;
          row_w[r] = w[a];
        }
      }
      if (valid) token_row[a] = r < R_cap ? r : -1;
    }
  }
}

// Exclusive scan of v[0..El) in place by one wave; returns the total.
__device__ __forceinline__ int wave_exclusive_scan(int *v, int El, int lane) {
  int carry = 0;
  for (int b = 0; b < El; b += 64) {
    int e = b + lane;
    int x = e < El ? v[e] : 0;
    int incl = x;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      int o = __shfl_up(incl, off, 64);
      if (lane >= off) incl += o;
    }
    if (e < El) v[e] = carry + incl - x;
    carry += __shfl(incl, 63, 64);
  }
  return carry;
}

// The whole permutation of N <= 8192 assignments by one workgroup of NW waves:
// counts, offsets, row_token / row_w and token_row.  smem holds (NW + 1) * El ints.
template <int NW>
__device__ __forceinline__ void permute_block(const int32_t *__restrict__ ids, const float *__restrict__ w, int N,
                                              int k, int lo, int El, int nbits, int R_cap,
                                              int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
                                              int32_t *__restrict__ row_token, float *__restrict__ row_w,
                                              int32_t *__restrict__ token_row, int *smem) {
  int *cnt = smem;             // [NW][El]: per-wave counts, then per-wave next row
  int *scan = smem + NW * El;  // [El]
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;  // NW waves of 64 lanes
  for (int i = threadIdx.x; i < NW * El; i += (NW * 64)) cnt[i] = 0;
  __syncthreads();
  const int per = ((N + (NW * 64) - 1) / (NW * 64)) * 64;  // multiple of 64
  const int a0 = min(N, wave * per), a1 = min(N, a0 + per);
  wave_count(ids, a0, a1, lo, El, nbits, cnt + wave * El, lane);
  __syncthreads();
  for (int e = threadIdx.x; e < El; e += (NW * 64)) {
    int s = 0;
    for (int v = 0; v < NW; v++) s += cnt[v * El + e];
    scan[e] = s;
    counts[e] = s;
  }
  __syncthreads();
  if (wave == 0) {
    int total = wave_exclusive_scan(scan, El, lane);
    if (lane == 0) offsets[El] = total;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < El; e += (NW * 64)) {
    int run = scan[e];
    offsets[e] = run;
    for (int v = 0; v < NW; v++) {
      int c = cnt[v * El + e];
      cnt[v * El + e] = run;
      run += c;
    }
  }
  __syncthreads();
  wave_assign(ids, w, a0, a1, k, lo, El, nbits, R_cap, cnt + wave * El, lane, row_token, row_w, token_row);
}

}  // namespace perm

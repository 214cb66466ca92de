// Local dispatch (moe_permute): per-expert counts, offsets and the stable
// grouping of assignments by expert, plus the optional row gather x -> x_perm.
//
// Dispatch groups every expert's tokens into the GEMM input buffers and, with
// replicated inputs, keeps only the tokens of the local experts ("Hosting Qwen
// on Blackwell", sections "MoE Dispatch - Combine" and "Expert parallelism");
// the per-expert row counts m_j are the AI-infra book's load measure (section
// 9.4.2) and the padding unit of the grouped GEMM (section 9.4.3).
//
// No host synchronisation anywhere.  Each wave owns a contiguous slice of the
// assignments in token-major order.  Pass 1 counts, per wave and expert, with a
// wave-wide "match" (lanes holding the same expert found with one ballot per
// expert-id bit) so only one lane per expert touches LDS.  A scan over experts
// and slices gives every wave its first row inside every expert.  Pass 2
// repeats the match and hands out rows by lane rank, which keeps the rows of
// one expert in increasing token order: the unique stable order.  Small
// batches run in one workgroup of 16 waves; large ones in chunks of 1024
// assignments (count kernel, one-workgroup scan of the chunk counts, assign
// kernel), the chunk counts living in the caller's workspace.
#include "permute_dev.h"

namespace {

using perm::kUnroll;
using perm::wave_count;
using perm::wave_assign;
using perm::wave_exclusive_scan;
using perm::match_lanes;
using perm::lanemask_lt;

constexpr int kPermWaves = 16;
constexpr int kPermThreads = kPermWaves * 64;
// Small batches: the whole problem in one workgroup of 16 waves.
__global__ __launch_bounds__(kPermThreads) void permute_kernel(const int32_t *__restrict__ ids,
                                                              const float *__restrict__ w, int N, int k, int lo,
                                                              int El, int nbits, int R_cap,
                                                              int32_t *__restrict__ counts,
                                                              int32_t *__restrict__ offsets,
                                                              int32_t *__restrict__ row_token,
                                                              float *__restrict__ row_w,
                                                              int32_t *__restrict__ token_row) {
  extern __shared__ int smem[];
  perm::permute_block<kPermWaves>(ids, w, N, k, lo, El, nbits, R_cap, counts, offsets, row_token, row_w, token_row,
                                  smem);
}

// Large batches: chunks of kChunk assignments, one 4-wave workgroup each.
constexpr int kChunkWaves = 4;
constexpr int kChunk = kChunkWaves * 64 * kUnroll / 2;  // 1024 assignments, 256 per wave

// Pass 1: per-chunk, per-expert counts -> cc[chunk][El].
__global__ __launch_bounds__(kChunkWaves * 64) void chunk_count_kernel(const int32_t *__restrict__ ids, int N, int lo,
                                                                       int El, int nbits, int32_t *__restrict__ cc) {
  extern __shared__ int smem[];  // [kChunkWaves][El]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < kChunkWaves * El; i += blockDim.x) smem[i] = 0;
  __syncthreads();
  const int a0 = min(N, blockIdx.x * kChunk + wave * (kChunk / kChunkWaves));
  const int a1 = min(N, a0 + kChunk / kChunkWaves);
  wave_count(ids, a0, a1, lo, El, nbits, smem + wave * El, lane);
  __syncthreads();
  for (int e = threadIdx.x; e < El; e += blockDim.x) {
    int s = 0;
    for (int v = 0; v < kChunkWaves; v++) s += smem[v * El + e];
    cc[(size_t)blockIdx.x * El + e] = s;
  }
}

// Pass 2 (one workgroup): counts and offsets from the chunk counts (read only).
__global__ __launch_bounds__(512) void chunk_scan_kernel(const int32_t *__restrict__ cc, int nchunks, int El,
                                                         int32_t *__restrict__ counts, int32_t *__restrict__ offsets) {
  extern __shared__ int smem[];  // [El]
  for (int e = threadIdx.x; e < El; e += blockDim.x) {
    int run = 0;
#pragma unroll 8
    for (int c = 0; c < nchunks; c++) run += cc[(size_t)c * El + e];
    smem[e] = run;
    counts[e] = run;
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    int total = wave_exclusive_scan(smem, El, threadIdx.x);
    if (threadIdx.x == 0) offsets[El] = total;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < El; e += blockDim.x) offsets[e] = smem[e];
}

// Pass 3: rows of each chunk, starting from its bases.
__global__ __launch_bounds__(kChunkWaves * 64) void chunk_assign_kernel(const int32_t *__restrict__ ids,
                                                                        const float *__restrict__ w, int N, int k,
                                                                        int lo, int El, int nbits, int R_cap,
                                                                        const int32_t *__restrict__ cc,
                                                                        const int32_t *__restrict__ offsets,
                                                                        int32_t *__restrict__ row_token,
                                                                        float *__restrict__ row_w,
                                                                        int32_t *__restrict__ token_row) {
  extern __shared__ int smem[];  // [kChunkWaves][El]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < kChunkWaves * El; i += blockDim.x) smem[i] = 0;
  __syncthreads();
  const int a0 = min(N, blockIdx.x * kChunk + wave * (kChunk / kChunkWaves));
  const int a1 = min(N, a0 + kChunk / kChunkWaves);
  wave_count(ids, a0, a1, lo, El, nbits, smem + wave * El, lane);
  __syncthreads();
  // first row of expert e in this chunk: offsets[e] + the counts of the chunks before it
  for (int e = threadIdx.x; e < El; e += blockDim.x) {
    int run = offsets[e];
#pragma unroll 8
    for (int c = 0; c < (int)blockIdx.x; c++) run += cc[(size_t)c * El + e];
    for (int v = 0; v < kChunkWaves; v++) {
      int c = smem[v * El + e];
      smem[v * El + e] = run;
      run += c;
    }
  }
  __syncthreads();
  wave_assign(ids, w, a0, a1, k, lo, El, nbits, R_cap, smem + wave * El, lane, row_token, row_w, token_row);
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

__global__ __launch_bounds__(256) void identity_rows_kernel(int T, int32_t *__restrict__ offsets,
                                                           int32_t *__restrict__ row_token, float *__restrict__ row_w) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < T) {
    row_token[i] = i;
    row_w[i] = 1.0f;
  }
  if (i == 0) {
    offsets[0] = 0;
    offsets[1] = T;
  }
}

}  // namespace

size_t permute_ws_bytes(int T, int k, int El) {
  const long long N = (long long)T * k;
  const long long nchunks = (N + kChunk - 1) / kChunk;
  return align_up(sizeof(int32_t) * (size_t)(nchunks > 0 ? nchunks : 1) * (size_t)El, 256);
}

hipError_t launch_permute(const int32_t *ids, const float *w, int T, int k, int lo, int El, int32_t *counts,
                          int32_t *offsets, int32_t *row_token, float *row_w, int32_t *token_row, int32_t *ws,
                          hipStream_t s) {
  int nbits = 0;
  while ((1 << nbits) < El) nbits++;
  const int N = T * k;
  const int R_cap = T * (k < El ? k : El);
  if (N <= 8192) {
    size_t shm = sizeof(int) * (size_t)(kPermWaves + 1) * El;
    hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(kPermThreads), shm, s, ids, w, N, k, lo, El, nbits, R_cap,
                       counts, offsets, row_token, row_w, token_row);
    return hipGetLastError();
  }
  const int nchunks = (N + kChunk - 1) / kChunk;
  const size_t shm = sizeof(int) * (size_t)kChunkWaves * El;
  hipLaunchKernelGGL(chunk_count_kernel, dim3(nchunks), dim3(kChunkWaves * 64), shm, s, ids, N, lo, El, nbits, ws);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(chunk_scan_kernel, dim3(1), dim3(512), sizeof(int) * (size_t)El, s, ws, nchunks, El, counts,
                     offsets);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL(chunk_assign_kernel, dim3(nchunks), dim3(kChunkWaves * 64), shm, s, ids, w, N, k, lo, El, nbits,
                     R_cap, ws, offsets, row_token, row_w, token_row);
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

hipError_t launch_identity_rows(int T, int32_t *offsets, int32_t *row_token, float *row_w, hipStream_t s) {
  const int grid = T > 0 ? (T + 255) / 256 : 1;
  hipLaunchKernelGGL(identity_rows_kernel, dim3(grid), dim3(256), 0, s, T, offsets, row_token, row_w);
  return hipGetLastError();
}

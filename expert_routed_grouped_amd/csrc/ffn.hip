// Grouped SwiGLU expert FFN (moe_grouped_ffn) for gfx950.
//
// Every local expert multiplies its own rows (a contiguous range of the
// grouped rows) by its gate/up and down matrices: a grouped GEMM over variable
// per-expert row counts (AI-infra book, section 9.4.3), with the expert shape
// of section 9.3.2 and the weighted combine of "Hosting Qwen on Blackwell",
// section "MoE Dispatch - Combine", fused into the down-projection epilogue.
//
// Work is cut into tiles of rows of one expert x output columns.  The tile
// list is never sent to the host: every workgroup finds its (expert, N tile,
// M tile) from the expert offsets on the device (a wave-wide prefix over the
// experts' M-tile counts).  The grid is sized for the worst case the host can
// bound (R_cap rows) and surplus workgroups exit at once; experts without rows
// get no tile and their weights are never read.  Consecutive tile numbers walk
// the M tiles of one (expert, N tile) first and are kept on one XCD, so the
// weight tile those M tiles share is fetched from HBM about once and served
// from that XCD's L2 afterwards.
//
// Two tile kernels, chosen by batch shape:
//  - few rows per expert (decode): the weight-streaming kernel of
//    ffn_stream.hip, bound by HBM bandwidth;
//  - many rows: the direct-to-LDS pipelined kernel of ffn_dma.hip, for bf16
//    weights and for e4m3 weights (codes copied into LDS, converted to bf16
//    exactly after the fragment reads, the per-output-channel scale applied in
//    the epilogue).
// fp32 weights take plain fp32 FMA loops (no matrix cores).
#include "ffn_common.h"

namespace {

using ffn::TileParams;

// ---------------------------------------------------------------------------
// fp32 path: plain fp32 FMA loops (small fp32 models; no matrix cores).
// ---------------------------------------------------------------------------
__device__ __forceinline__ int expert_of_row(const int32_t *offsets, int El, int r) {
  int lo = 0, hi = El - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (offsets[mid] <= r) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

__global__ __launch_bounds__(64) void gate_up_f32_kernel(const float *__restrict__ a, int gather,
                                                         const int32_t *__restrict__ offsets,
                                                         const int32_t *__restrict__ row_token, int El, int H, int I,
                                                         const float *__restrict__ w, float *__restrict__ h) {
  const int r = blockIdx.x;  // grid = R_cap rows
  if (r >= offsets[El]) return;
  const int i = blockIdx.y * 64 + threadIdx.x;
  if (i >= I) return;
  const int e = expert_of_row(offsets, El, r);
  const float *src = a + (size_t)(gather ? row_token[r] : r) * H;
  const float *wg = w + ((size_t)e * 2 * I + i) * H;
  const float *wu = w + ((size_t)e * 2 * I + I + i) * H;
  float g = 0.f, u = 0.f;
  for (int k = 0; k < H; k++) {
    g = __builtin_fmaf(src[k], wg[k], g);
    u = __builtin_fmaf(src[k], wu[k], u);
  }
  h[(size_t)r * I + i] = silu_f32(g) * u;
}

__global__ __launch_bounds__(64) void down_f32_kernel(const float *__restrict__ h, const int32_t *__restrict__ offsets,
                                                      const int32_t *__restrict__ row_token,
                                                      const float *__restrict__ row_w, int El, int H, int I,
                                                      const float *__restrict__ w, float *__restrict__ y,
                                                      float *__restrict__ y_perm) {
  const int r = blockIdx.x;  // grid = R_cap rows
  if (r >= offsets[El]) return;
  const int n = blockIdx.y * 64 + threadIdx.x;
  if (n >= H) return;
  const int e = expert_of_row(offsets, El, r);
  const float *hr = h + (size_t)r * I;
  const float *wd = w + ((size_t)e * H + n) * I;
  float o = 0.f;
  for (int i = 0; i < I; i++) o = __builtin_fmaf(hr[i], wd[i], o);
  if (y != nullptr) atomicAdd(y + (size_t)row_token[r] * H + n, row_w[r] * o);
  else y_perm[(size_t)r * H + n] = o;
}

}  // namespace

namespace {

// One thread moves one 16-byte piece of a weight row to its place in the packed layout.
__global__ void pack_weights_kernel(const char *__restrict__ w, int esz, size_t rows, int K, char *__restrict__ out) {
  const size_t per_row = (size_t)K * esz / 16;
  const size_t n = rows * per_row;
  for (size_t u = (size_t)blockIdx.x * blockDim.x + threadIdx.x; u < n; u += (size_t)gridDim.x * blockDim.x) {
    const size_t row = u / per_row;
    const int kb = (int)(u - row * per_row) * 16;  // byte offset inside the row-major row
    const int k = kb / esz;
    const size_t dst =
        ffn::w_piece_off(1, row, (kb % (64 * esz)) / 16, K, esz) + (size_t)(k >> 6) * ffn::w_chunk_step(1, esz);
    *(u32x4_t *)(out + dst) = *(const u32x4_t *)(w + row * (size_t)K * esz + kb);
  }
}

}  // namespace

hipError_t launch_pack_weights(const void *w, int esz, int E, int N, int K, void *packed, hipStream_t s) {
  const size_t rows = (size_t)E * N;
  const size_t n = rows * ((size_t)K * esz / 16);
  if (n == 0) return hipSuccess;
  const size_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(pack_weights_kernel, dim3(blocks < 8192 ? (unsigned)blocks : 8192u), dim3(256), 0, s,
                     (const char *)w, esz, rows, K, (char *)packed);
  return hipGetLastError();
}

hipError_t launch_ffn(const FfnArgs &a, hipStream_t s) {
  hipError_t err;
  if (a.R_cap == 0 || a.T == 0) return hipSuccess;
  const bool first = a.phase & 1, second = a.phase & 2;
  if (a.w_dt == 0) {  // fp32
    dim3 g1(a.R_cap, ceil_div_i(a.I, 64)), g2(a.R_cap, ceil_div_i(a.H, 64));
    if (first) {
      hipLaunchKernelGGL(gate_up_f32_kernel, g1, dim3(64), 0, s, (const float *)a.a, a.gather, a.offsets,
                         a.row_token, a.El, a.H, a.I, (const float *)a.w_gu, (float *)a.h);
      if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    if (second) {
      hipLaunchKernelGGL(down_f32_kernel, g2, dim3(64), 0, s, (const float *)a.h, a.offsets, a.row_token, a.row_w,
                         a.El, a.H, a.I, (const float *)a.w_d, a.y, a.y_perm);
      if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    return hipSuccess;
  }
  // Few rows per expert on average: stream the weights (HBM bound); else tiles (matrix-core bound).
  const bool stream = a.kernel == 1 || (a.kernel == 0 && (long long)a.R_cap <= 48LL * a.El);
  TileParams base{};
  base.offsets = a.offsets;
  base.row_token = a.row_token;
  base.row_w = a.row_w;
  base.El = a.El;
  base.H = a.H;
  base.I = a.I;
  base.R_cap = a.R_cap;
  base.wpacked = a.wpacked;
  return stream ? launch_ffn_stream(base, a, s) : launch_ffn_dma(base, a, s);
}


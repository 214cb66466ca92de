// Grouped SwiGLU expert FFN (moe_grouped_ffn) for gfx950.
//
// Every local expert multiplies its own rows (a contiguous range of the
// grouped rows) by its gate/up and down matrices: a grouped GEMM over variable
// per-expert row counts (AI-infra book, section 9.4.3), with the expert shape
// of section 9.3.2 and the weighted combine of "Hosting Qwen on Blackwell",
// section "MoE Dispatch - Combine", fused into the down-projection epilogue.
//
// Work is cut into tiles of BM rows of one expert x BN output columns.  The
// tile list is never sent to the host: a one-workgroup schedule kernel turns
// the per-expert row counts into a prefix of M-tiles, and every GEMM workgroup
// finds its (expert, N-tile, M-tile) by a binary search of that prefix.  The
// grid is sized for the worst case the host can bound (R_cap rows) and surplus
// workgroups exit at once; experts without rows get no tile and their weights
// are never read.  Consecutive tile numbers walk the M-tiles of one (expert,
// N-tile) first and are kept on one XCD, so the weight tile those M-tiles share
// is fetched from HBM about once and served from that XCD's L2 afterwards.
//
// Inside a tile: bf16 operands are staged through LDS (global -> registers ->
// LDS, two LDS stages, one barrier per K step) in rows of 64 k-elements with
// the 16-byte chunks XOR-swizzled by row, so the 16-byte MFMA operand reads of
// a wave hit distinct banks.  fp8 e4m3 weights are converted to bf16 (exact)
// on their way into LDS, so the MFMA loop is the same for both weight types
// and the per-output-channel scale is applied in the epilogue.  Four waves
// each own a 64 x 64 quarter of the 128 x 128 tile as 2 x 2 blocks of
// v_mfma_f32_32x32x16_bf16 with fp32 accumulation.
#include "common.h"

namespace {

constexpr int BM = 128, BN = 128, BK = 64, NTHR = 256;
constexpr int LDS_TILE = BM * BK * 2;  // bytes of one A (or B) stage

struct TileParams {
  const void *a;          // activations: x [T,H] (gather) / x_perm [R_cap,H] (gate-up), h [R_cap,I] (down)
  const int32_t *offsets; // [El+1]
  const int32_t *row_token;
  const float *row_w;
  const void *w;          // this projection's weights [El, Nw, K]
  const float *scale;     // [El, Nw] (fp8 only)
  void *out;              // h [R_cap,I] bf16 (gate-up) / y [T,H] or y_perm [R_cap,H] fp32 (down)
  const int32_t *sched;   // M-tile prefix [El+1]
  int El, H, I;
  int R_cap;              // rows past R_cap are never touched, whatever the offsets say
};

__device__ __forceinline__ int lds_off(int row, int chunk) { return row * 128 + ((chunk ^ (row & 7)) << 4); }

// Locate this workgroup's tile.  Returns false for surplus workgroups.
__device__ __forceinline__ bool find_tile(const TileParams &p, int NT, int &e, int &nt, int &r0, int &rows) {
  const int total = p.sched[p.El] * NT;
  const int bid = blockIdx.x;
  if (bid >= total) return false;
  // Keep consecutive tile numbers on one XCD (workgroups go round-robin over 8 XCDs).
  const int xcd = bid & 7, j = bid >> 3, q = total >> 3, rem = total & 7;
  const int L = xcd * q + min(xcd, rem) + j;
  int lo = 0, hi = p.El - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (p.sched[mid] * NT <= L) lo = mid;
    else hi = mid - 1;
  }
  e = lo;
  const int mtiles = p.sched[e + 1] - p.sched[e];
  const int rr = L - p.sched[e] * NT;
  nt = rr / mtiles;
  const int mt = rr - nt * mtiles;
  r0 = p.offsets[e] + mt * BM;
  rows = min(BM, min(p.offsets[e + 1], p.R_cap) - r0);
  return rows > 0;
}

// MODE 0: gate/up + SwiGLU -> h (bf16).  MODE 1: down + combine epilogue.
// FP8: weights are e4m3 codes.  GATHER (mode 0): A row r is a[row_token[r]].
// ATOMIC (mode 1): y[row_token[r]] += row_w[r] * o, else y_perm[r] = o.
template <int MODE, bool FP8, bool GATHER, bool ATOMIC>
__global__ __launch_bounds__(NTHR, 2) void ffn_tile_kernel(TileParams p) {
  __shared__ __attribute__((aligned(16))) char lds[2][2][LDS_TILE];  // [stage][A/B]
  const int K = MODE == 0 ? p.H : p.I;
  const int Nw = MODE == 0 ? 2 * p.I : p.H;  // weight rows per expert
  const int NT = MODE == 0 ? p.I / 64 : (p.H + BN - 1) / BN;
  int e, nt, r0, rows;
  if (!find_tile(p, NT, e, nt, r0, rows)) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- A sources: this thread stages chunk (tid & 7) of rows (tid >> 3) + 32q
  const int ach = tid & 7;
  const uint16_t *asrc[4];
#pragma unroll
  for (int q = 0; q < 4; q++) {
    int m = (tid >> 3) + 32 * q;
    int r = r0 + min(m, rows - 1);
    size_t src_row = (MODE == 0 && GATHER) ? (size_t)p.row_token[r] : (size_t)r;
    asrc[q] = (const uint16_t *)p.a + src_row * K + ach * 8;
  }
  // ---- B sources
  constexpr int BQ = FP8 ? 2 : 4;  // 16-byte global chunks per thread per K step
  const char *bsrc[BQ];
#pragma unroll
  for (int q = 0; q < BQ; q++) {
    int rho, ch;
    if constexpr (FP8) { rho = (tid >> 2) + 64 * q; ch = tid & 3; }
    else { rho = (tid >> 3) + 32 * q; ch = tid & 7; }
    int wrow;
    if constexpr (MODE == 0) wrow = ((rho >> 5) & 1) * p.I + nt * 64 + (rho >> 6) * 32 + (rho & 31);
    else wrow = min(nt * BN + rho, p.H - 1);
    size_t esz = FP8 ? 1 : 2;
    bsrc[q] = (const char *)p.w + (((size_t)e * Nw + wrow) * K) * esz + ch * 16;
  }

  u32x4_t areg[4], breg[BQ];
  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int j = 0; j < 2; j++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[i][j][r] = 0.0f;

  const int KT = K / BK;
  for (int kt = -1; kt < KT; kt++) {
    // global -> registers for step kt+1 (in flight while step kt computes)
    if (kt + 1 < KT) {
      const int k0 = (kt + 1) * BK;
#pragma unroll
      for (int q = 0; q < 4; q++) areg[q] = *(const u32x4_t *)(asrc[q] + k0);
#pragma unroll
      for (int q = 0; q < BQ; q++) breg[q] = *(const u32x4_t *)(bsrc[q] + (size_t)k0 * (FP8 ? 1 : 2));
    }
    if (kt >= 0) {
      const char *A = lds[kt & 1][0], *B = lds[kt & 1][1];
#pragma unroll
      for (int kk = 0; kk < 4; kk++) {
        const int ch = kk * 2 + (lane >> 5);
        bf16x8_t af[2], bfr[2];
#pragma unroll
        for (int f = 0; f < 2; f++) {
          af[f] = *(const bf16x8_t *)(A + lds_off(wm * 64 + f * 32 + (lane & 31), ch));
          bfr[f] = *(const bf16x8_t *)(B + lds_off(wn * 64 + f * 32 + (lane & 31), ch));
        }
#pragma unroll
        for (int i = 0; i < 2; i++)
#pragma unroll
          for (int j = 0; j < 2; j++)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
      }
    }
    // registers -> LDS stage (kt+1)&1; the barrier at the end of step kt-1 made
    // sure nobody still reads that stage
    if (kt + 1 < KT) {
      char *A = lds[(kt + 1) & 1][0], *B = lds[(kt + 1) & 1][1];
#pragma unroll
      for (int q = 0; q < 4; q++) *(u32x4_t *)(A + lds_off((tid >> 3) + 32 * q, ach)) = areg[q];
#pragma unroll
      for (int q = 0; q < BQ; q++) {
        if constexpr (FP8) {
          const int rho = (tid >> 2) + 64 * q, ch = tid & 3;
          uint2 c0 = e4m3x4_to_bf16x4(breg[q].x), c1 = e4m3x4_to_bf16x4(breg[q].y);
          uint2 c2 = e4m3x4_to_bf16x4(breg[q].z), c3 = e4m3x4_to_bf16x4(breg[q].w);
          *(uint4 *)(B + lds_off(rho, 2 * ch)) = make_uint4(c0.x, c0.y, c1.x, c1.y);
          *(uint4 *)(B + lds_off(rho, 2 * ch + 1)) = make_uint4(c2.x, c2.y, c3.x, c3.y);
        } else {
          *(u32x4_t *)(B + lds_off((tid >> 3) + 32 * q, tid & 7)) = breg[q];
        }
      }
    }
    __syncthreads();
  }

  // ---- epilogue.  acc[i][j][r] at lane l is row wm*64 + i*32 + 8*(r/4) + 4*(l/32) + r%4,
  // column wn*64 + j*32 + l%32 of the tile.
  if constexpr (MODE == 0) {
    const int col = nt * 64 + wn * 32 + (lane & 31);  // intermediate index i
    float sg = 1.0f, su = 1.0f;
    if constexpr (FP8) {
      sg = p.scale[(size_t)e * Nw + col];
      su = p.scale[(size_t)e * Nw + p.I + col];
    }
    uint16_t *hout = (uint16_t *)p.out;
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int m = wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (m < rows) {
          const float g = acc[i][0][r] * sg, u = acc[i][1][r] * su;
          hout[(size_t)(r0 + m) * p.I + col] = f32_to_bf16(silu_f32(g) * u);
        }
      }
  } else {
    float *out = (float *)p.out;
#pragma unroll
    for (int j = 0; j < 2; j++) {
      const int n = nt * BN + wn * 64 + j * 32 + (lane & 31);
      if (n >= p.H) continue;
      const float sc = FP8 ? p.scale[(size_t)e * Nw + n] : 1.0f;
#pragma unroll
      for (int i = 0; i < 2; i++)
#pragma unroll
        for (int r = 0; r < 16; r++) {
          const int m = wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          if (m < rows) {
            const int row = r0 + m;
            const float o = acc[i][j][r] * sc;
            if constexpr (ATOMIC) {
              atomicAdd(out + (size_t)p.row_token[row] * p.H + n, p.row_w[row] * o);
            } else {
              out[(size_t)row * p.H + n] = o;
            }
          }
        }
    }
  }
}

// sched[e] = number of BM-row tiles of experts < e (exclusive prefix), sched[El] = total.
__global__ __launch_bounds__(64) void schedule_kernel(const int32_t *__restrict__ offsets, int El, int bm,
                                                      int32_t *__restrict__ sched) {
  const int lane = threadIdx.x;
  int carry = 0;
  for (int b = 0; b < El; b += 64) {
    int e = b + lane;
    int v = e < El ? (offsets[e + 1] - offsets[e] + bm - 1) / bm : 0;
    int incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      int o = __shfl_up(incl, off, 64);
      if (lane >= off) incl += o;
    }
    if (e < El) sched[e] = carry + incl - v;
    carry += __shfl(incl, 63, 64);
  }
  if (lane == 0) sched[El] = carry;
}

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

template <int MODE, bool FP8, bool GATHER, bool ATOMIC>
hipError_t launch_tile(const TileParams &tp, int grid, hipStream_t s) {
  hipLaunchKernelGGL((ffn_tile_kernel<MODE, FP8, GATHER, ATOMIC>), dim3(grid), dim3(NTHR), 0, s, tp);
  return hipGetLastError();
}

}  // namespace

size_t ffn_sched_bytes(int El) { return align_up(sizeof(int32_t) * (size_t)(El + 1), 256); }

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
  if (first) {
    hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(64), 0, s, a.offsets, a.El, BM, a.sched);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  // worst-case M-tiles: sum_e ceil(c_e/BM) <= (R + El*(BM-1))/BM and <= El*ceil(T/BM)
  long long mt1 = ((long long)a.R_cap + (long long)a.El * (BM - 1)) / BM;
  long long mt2 = (long long)a.El * ceil_div_i(a.T, BM);
  long long max_mt = mt1 < mt2 ? mt1 : mt2;
  const bool fp8 = a.w_dt == 2;
  TileParams tp{};
  tp.offsets = a.offsets;
  tp.row_token = a.row_token;
  tp.row_w = a.row_w;
  tp.sched = a.sched;
  tp.El = a.El;
  tp.H = a.H;
  tp.I = a.I;
  tp.R_cap = a.R_cap;
  // gate/up
  tp.a = a.a;
  tp.w = a.w_gu;
  tp.scale = a.s_gu;
  tp.out = a.h;
  int grid1 = (int)(max_mt * (a.I / 64));
  if (first) {
    if (fp8) err = a.gather ? launch_tile<0, true, true, false>(tp, grid1, s) : launch_tile<0, true, false, false>(tp, grid1, s);
    else err = a.gather ? launch_tile<0, false, true, false>(tp, grid1, s) : launch_tile<0, false, false, false>(tp, grid1, s);
    if (err != hipSuccess) return err;
  }
  if (!second) return hipSuccess;
  // down
  tp.a = a.h;
  tp.w = a.w_d;
  tp.scale = a.s_d;
  const bool atomic = a.y != nullptr;
  tp.out = atomic ? (void *)a.y : (void *)a.y_perm;
  int grid2 = (int)(max_mt * ceil_div_i(a.H, BN));
  if (fp8) err = atomic ? launch_tile<1, true, false, true>(tp, grid2, s) : launch_tile<1, true, false, false>(tp, grid2, s);
  else err = atomic ? launch_tile<1, false, false, true>(tp, grid2, s) : launch_tile<1, false, false, false>(tp, grid2, s);
  return err;
}

// Weight-streaming grouped FFN for small batches (decode).
//
// With a few rows per expert the layer is bound by reading each active
// expert's weights from HBM once (AI-infra book, section 9.3.3: 64 tokens x
// top-8 touch about 126 of 128 experts, ~4.4 GiB of bf16 weights for 19.3
// GFLOP; "Hosting Qwen on Blackwell", section "Decoders": small-batch GEMMs are
// limited by moving weights from HBM to the matrix units).  The design goal is
// therefore bytes in flight, not reuse:
//
//  - no LDS and no barriers: every wave is independent and owns 32 output
//    columns of one expert (32 gate + 32 up rows for the gate/up half) for up to
//    64 rows of that expert (two 32-row MFMA blocks);
//  - the wave streams its weight rows straight from HBM into registers in the
//    operand layout of v_mfma_f32_32x32x16_bf16 (stream_core.h: every lane reads
//    64 contiguous bytes of one row per 64-wide k chunk, two chunks in flight);
//    the activations are read with the same layout (they are small and stay in
//    L2), and many waves per CU cover the HBM latency.
//
// Tiles are located the same way as in the tile kernels (64-row M tiles, found
// from the expert offsets on the device); an expert with more than 64 rows gets
// more M tiles and its weights are streamed once per M tile, which is still
// correct.
#include "ffn_common.h"
#include "stream_core.h"

namespace {

using ffn::TileParams;

#ifndef STREAM_MB
#define STREAM_MB 2
#endif
constexpr int SMB = STREAM_MB;  // 32-row MFMA blocks per M tile
constexpr int SBM = 32 * SMB;   // rows per M tile
constexpr int SWAVES = 4;   // waves per block, 32 output columns each
constexpr int SCOLS = 32 * SWAVES;  // gate/up columns per block (down: twice as many)

template <int MODE, bool FP8, bool GATHER, bool ATOMIC>
__global__ __launch_bounds__(64 * SWAVES) void ffn_stream_kernel(TileParams p) {
  const int K = MODE == 0 ? p.H : p.I;
  const int Ncols = MODE == 0 ? p.I : p.H;
  const int Nw = MODE == 0 ? 2 * p.I : p.H;
  constexpr int WCOLS = MODE == 0 ? 32 : 64;  // output columns per wave
  const int NT = (Ncols + SWAVES * WCOLS - 1) / (SWAVES * WCOLS);
  const int KS = p.ksplit > 1 ? p.ksplit : 1;  // K slices: tile "column" index = nt * KS + slice
  int e, ntk, r0, rows;
  if (!ffn::find_tile<SBM>(p, NT * KS, e, ntk, r0, rows)) return;
  const int nt = ntk / KS, ks = ntk - nt * KS;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c0 = (nt * SWAVES + wave) * WCOLS;
  if (c0 >= Ncols) return;  // Ncols is a multiple of 64: a wave's columns are all valid or all past the end
  const int n = lane & 31, g = lane >> 5;
  constexpr int NB = 2;                  // weight row blocks per wave: gate + up, or two down blocks
  const bool two_m = SMB > 1 && rows > 32;  // wave-uniform

  // weight rows of this lane (k offset 32g inside every 64-wide chunk)
  const size_t wesz = FP8 ? 1 : 2;
  const char *wrow[NB];
  const size_t cstep = ffn::w_chunk_step(p.wpacked, (int)wesz);  // bytes from one 64-wide k chunk to the next
  {
    const size_t r0w = (size_t)e * Nw + c0 + n;                 // this lane's first weight row
    const size_t r1w = MODE == 0 ? r0w + p.I : r0w + 32;        // up row / second down block
    wrow[0] = (const char *)p.w + ffn::w_piece_off(p.wpacked, r0w, 2 * (int)wesz * g, K, (int)wesz);
    wrow[1] = (const char *)p.w + ffn::w_piece_off(p.wpacked, r1w, 2 * (int)wesz * g, K, (int)wesz);
  }
  // activation rows (two 32-row blocks; rows past the end repeat the last valid row)
  const uint16_t *arow[SMB];
#pragma unroll
  for (int mb = 0; mb < SMB; mb++) {
    const int r = r0 + min(mb * 32 + n, rows - 1);
    const size_t src = (MODE == 0 && GATHER) ? (size_t)p.row_token[r] : (size_t)r;
    arow[mb] = (const uint16_t *)p.a + src * K + 32 * g;
  }

  f32x16_t acc[SMB][NB];
  sc::zero_acc(acc);
  // this workgroup's 64-wide k chunks: [kb, kb + KC) of the K / 64 (K is a multiple of 64)
  const int kb = ks * (K / 64) / KS;
  const int KC = (ks + 1) * (K / 64) / KS - kb;
#pragma unroll
  for (int b = 0; b < NB; b++) wrow[b] += (size_t)kb * cstep;
#pragma unroll
  for (int mb = 0; mb < SMB; mb++) arow[mb] += (size_t)kb * 64;
  sc::stream_mfma<FP8, SMB, NB>(wrow, ffn::w_lane_piece_step(p.wpacked, (int)wesz), cstep, arow, two_m, KC, acc);

  // ---- epilogue: acc[mb][b][r] at lane l is row mb*32 + 8*(r/4) + 4*(l/32) + r%4, column c0 + l%32
  const int col = c0 + n;
  if constexpr (MODE == 0) {
    float sg = 1.0f, su = 1.0f;
    if constexpr (FP8) {
      sg = p.scale[(size_t)e * Nw + col];
      su = p.scale[(size_t)e * Nw + p.I + col];
    }
    uint16_t *hout = (uint16_t *)p.out;
#pragma unroll
    for (int mb = 0; mb < SMB; mb++) {
      if (mb == 1 && !two_m) break;
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int m = mb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
        if (m < rows) {
          const float gt = acc[mb][0][r] * sg, u = acc[mb][1][r] * su;
          if (KS > 1) {  // partial sums of one K slice; SwiGLU runs once they are complete
            atomicAdd(p.gu32 + (size_t)(r0 + m) * 2 * p.I + col, gt);
            atomicAdd(p.gu32 + (size_t)(r0 + m) * 2 * p.I + p.I + col, u);
          } else {
            hout[(size_t)(r0 + m) * p.I + col] = f32_to_bf16(silu_fast(gt) * u);
          }
        }
      }
    }
  } else {
    float *out = (float *)p.out;
#pragma unroll
    for (int b = 0; b < NB; b++) {
      const int cb = col + 32 * b;
      const float sc = FP8 ? p.scale[(size_t)e * Nw + cb] : 1.0f;
#pragma unroll
      for (int mb = 0; mb < SMB; mb++) {
        if (mb == 1 && !two_m) break;
#pragma unroll
        for (int r = 0; r < 16; r++) {
          const int m = mb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
          if (m < rows) {
            const int row = r0 + m;
            const float o = acc[mb][b][r] * sc;
            if constexpr (ATOMIC) atomicAdd(out + (size_t)p.row_token[row] * p.H + cb, p.row_w[row] * o);
            else out[(size_t)row * p.H + cb] = o;
          }
        }
      }
    }
  }
}

// h = bf16(silu(G) * U) from the completed K-slice sums (rows < R_cap, 8 columns per thread).
__global__ __launch_bounds__(256) void swiglu_rows_kernel(const float *__restrict__ gu32, int rows, int I,
                                                          uint16_t *__restrict__ h) {
  const int per_row = I / 8;
  const size_t n = (size_t)rows * per_row;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
    const size_t r = i / per_row;
    const int c = (int)(i - r * per_row) * 8;
    const float *g = gu32 + r * 2 * I + c;
    uint16_t o[8];
#pragma unroll
    for (int j = 0; j < 8; j++) o[j] = f32_to_bf16(silu_fast(g[j]) * g[I + j]);
    *(u32x4_t *)(h + r * I + c) = u32x4_t{o[0] | ((uint32_t)o[1] << 16), o[2] | ((uint32_t)o[3] << 16),
                                         o[4] | ((uint32_t)o[5] << 16), o[6] | ((uint32_t)o[7] << 16)};
  }
}

template <int MODE, bool FP8, bool GATHER, bool ATOMIC>
hipError_t launch_s(const TileParams &tp, int grid, hipStream_t s) {
  hipLaunchKernelGGL((ffn_stream_kernel<MODE, FP8, GATHER, ATOMIC>), dim3(grid), dim3(64 * SWAVES), 0, s, tp);
  return hipGetLastError();
}

}  // namespace

int ffn_stream_bm() { return SBM; }

// Both halves (or one, per ``phase``) of the streaming FFN.
hipError_t launch_ffn_stream(const TileParams &base, const FfnArgs &a, hipStream_t s) {
  hipError_t err = hipSuccess;
  const long long mt1 = ((long long)a.R_cap + (long long)a.El * (SBM - 1)) / SBM;
  const long long mt2 = (long long)a.El * ceil_div_i(a.T, SBM);
  const long long max_mt = mt1 < mt2 ? mt1 : mt2;
  const bool fp8 = a.w_dt == 2;
  TileParams tp = base;
  // split K only with the fused combine (partial down-projection sums add straight into y)
  const int ks = (a.ksplit > 1 && a.y != nullptr && a.gu32 != nullptr) ? a.ksplit : 1;
  tp.ksplit = ks;
  tp.gu32 = a.gu32;
  if (a.phase & 1) {
    tp.a = a.a;
    tp.w = a.w_gu;
    tp.scale = a.s_gu;
    tp.out = a.h;
    if (ks > 1 && (err = launch_zero_f32(a.gu32, (size_t)a.R_cap * 2 * a.I, s)) != hipSuccess) return err;
    const int grid = (int)(max_mt * ceil_div_i(a.I, SCOLS) * ks);
    if (fp8) err = a.gather ? launch_s<0, true, true, false>(tp, grid, s) : launch_s<0, true, false, false>(tp, grid, s);
    else err = a.gather ? launch_s<0, false, true, false>(tp, grid, s) : launch_s<0, false, false, false>(tp, grid, s);
    if (err != hipSuccess) return err;
    if (ks > 1) {
      const size_t n = (size_t)a.R_cap * (a.I / 8);
      const int g = (int)((n + 255) / 256 < 2048 ? (n + 255) / 256 : 2048);
      hipLaunchKernelGGL(swiglu_rows_kernel, dim3(g > 0 ? g : 1), dim3(256), 0, s, a.gu32, a.R_cap, a.I,
                         (uint16_t *)a.h);
      if ((err = hipGetLastError()) != hipSuccess) return err;
    }
  }
  if (a.phase & 2) {
    tp.a = a.h;
    tp.w = a.w_d;
    tp.scale = a.s_d;
    const bool atomic = a.y != nullptr;
    tp.out = atomic ? (void *)a.y : (void *)a.y_perm;
    tp.ksplit = ks > 1 ? (ks < a.I / 64 ? ks : a.I / 64) : 1;  // at most one 64-wide chunk per slice
    const int grid = (int)(max_mt * ceil_div_i(a.H, 2 * SCOLS) * tp.ksplit);  // down: 64 columns per wave
    if (fp8) err = atomic ? launch_s<1, true, false, true>(tp, grid, s) : launch_s<1, true, false, false>(tp, grid, s);
    else err = atomic ? launch_s<1, false, false, true>(tp, grid, s) : launch_s<1, false, false, false>(tp, grid, s);
  }
  return err;
}

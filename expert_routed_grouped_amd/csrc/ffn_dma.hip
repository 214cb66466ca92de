// Grouped FFN tiles for large batches with bf16 weights: operands move from
// HBM/L2 straight into LDS (global_load_lds, no register staging) through a
// four-stage ring, three K steps ahead of the matrix cores.
//
// Tile: 256 rows of one expert x 256 weight rows, K step 32; eight waves as
// 2 (M) x 4 (N), each wave 128 rows x 64 weight rows = 4 x 2 blocks of
// v_mfma_f32_32x32x16_bf16 (fp32 accumulation).  Gate/up tiles hold the gate
// rows and the up rows of the same 128 intermediate columns, so the SwiGLU
// epilogue finds G and U of one output in the same lane and register.
//
// LDS rows are 32 bf16 = four 16-byte chunks; chunk c of row r sits in slot
// c ^ ((r >> 2) & 3), which keeps the 16 lanes of one LDS cycle on 16 distinct
// 16-byte bank groups when they read one chunk of 16 consecutive rows.  A
// global_load_lds writes the 16 bytes of lane i to slot i of a 1 KB segment, so
// every lane fetches the global chunk that belongs to its slot.
//
// Synchronisation per K step kt: wait for this wave's own loads of step kt
// (vmcnt), one barrier (all waves' loads of kt have landed and nobody still
// reads the stage about to be refilled), issue the loads of step kt+3, run the
// MFMAs of step kt.  The waits are explicit because the barrier used here
// carries no memory fence (a fence would drain every load still in flight).
//
// Rows past the expert's count are never multiplied: the K loop is
// instantiated for 0..4 active 32-row blocks per wave.
#include "ffn_common.h"

namespace {

using ffn::TileParams;

constexpr int BM = 256, BN = 256, BK = 32, NTHR = 512, STAGES = 4;
constexpr int A_BYTES = BM * BK * 2;           // 16 KB
constexpr int STAGE_BYTES = A_BYTES + BN * BK * 2;  // 32 KB

__device__ __forceinline__ int lds_off32(int row, int chunk) { return row * 64 + ((chunk ^ ((row >> 2) & 3)) << 4); }

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ void barrier_no_fence() { asm volatile("s_barrier" ::: "memory"); }

// wait until at most n of this wave's vector-memory operations are in flight
__device__ __forceinline__ void wait_vm(int n) {
  if (n >= 8) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  else if (n >= 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

struct DmaSrc {
  uint32_t aoff[2], boff[2];  // byte offsets of this lane's two A and two B segments (step 0)
};

template <int NMB>
__device__ __forceinline__ void dma_kloop(const char *abase, const char *bbase, const DmaSrc &src, int K, int wave,
                                          int lane, int wm, int wn, char (*lds)[STAGE_BYTES],
                                          f32x16_t (&acc)[NMB > 0 ? NMB : 1][2]) {
  const int KT = K / BK;
  // this wave fills 1 KB segments 2*wave and 2*wave+1 of the A part and of the B part
  auto issue = [&](int kt) __attribute__((always_inline)) {
    char *st = lds[kt % STAGES];
    const size_t k0b = (size_t)kt * BK * 2;
#pragma unroll
    for (int u = 0; u < 2; u++) {
      __builtin_amdgcn_global_load_lds((const void *)(abase + k0b + src.aoff[u]),
                                       (lds_void *)(st + (2 * wave + u) * 1024), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void *)(bbase + k0b + src.boff[u]),
                                       (lds_void *)(st + A_BYTES + (2 * wave + u) * 1024), 16, 0, 0);
    }
  };
  issue(0);
  if (KT > 1) issue(1);
  if (KT > 2) issue(2);
  for (int kt = 0; kt < KT; kt++) {
    wait_vm(4 * min(2, KT - 1 - kt));
    barrier_no_fence();
    if (kt + 3 < KT) issue(kt + 3);
    if constexpr (NMB > 0) {
      const char *A = lds[kt % STAGES], *B = A + A_BYTES;
#pragma unroll
      for (int kk = 0; kk < 2; kk++) {
        const int ch = kk * 2 + (lane >> 5);
        bf16x8_t bf[2], af[NMB];
#pragma unroll
        for (int j = 0; j < 2; j++) bf[j] = *(const bf16x8_t *)(B + lds_off32(wn * 64 + j * 32 + (lane & 31), ch));
#pragma unroll
        for (int i = 0; i < NMB; i++) af[i] = *(const bf16x8_t *)(A + lds_off32(wm * 128 + i * 32 + (lane & 31), ch));
#pragma unroll
        for (int i = 0; i < NMB; i++)
#pragma unroll
          for (int j = 0; j < 2; j++) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
      }
    }
  }
}

template <int MODE, bool ATOMIC, int NMB>
__device__ __forceinline__ void dma_body(const TileParams &p, const char *abase, const char *bbase, const DmaSrc &src,
                                         int K, int nt, int r0, int mvalid, int wave, int lane, int wm, int wn,
                                         char (*lds)[STAGE_BYTES]) {
  constexpr int NA = NMB > 0 ? NMB : 1;
  f32x16_t acc[NA][2];
#pragma unroll
  for (int i = 0; i < NA; i++)
#pragma unroll
    for (int j = 0; j < 2; j++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[i][j][r] = 0.0f;
  dma_kloop<NMB>(abase, bbase, src, K, wave, lane, wm, wn, lds, acc);
  if constexpr (NMB > 0) {
    // acc[i][j][r] at lane l is row wm*128 + i*32 + 8*(r/4) + 4*(l/32) + r%4,
    // weight row wn*64 + j*32 + l%32 of the tile
    if constexpr (MODE == 0) {
      if (nt * 128 + wn * 32 >= p.I) return;
      const int col = nt * 128 + wn * 32 + (lane & 31);  // intermediate index
      uint16_t *hout = (uint16_t *)p.out;
#pragma unroll
      for (int i = 0; i < NA; i++)
#pragma unroll
        for (int r = 0; r < 16; r++) {
          const int m = i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          if (m < mvalid)
            hout[(size_t)(r0 + wm * 128 + m) * p.I + col] = f32_to_bf16(silu_f32(acc[i][0][r]) * acc[i][1][r]);
        }
    } else {
      float *out = (float *)p.out;
#pragma unroll
      for (int j = 0; j < 2; j++) {
        const int n = nt * BN + wn * 64 + j * 32 + (lane & 31);
        if (n >= p.H) continue;
#pragma unroll
        for (int i = 0; i < NA; i++)
#pragma unroll
          for (int r = 0; r < 16; r++) {
            const int m = i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            if (m < mvalid) {
              const int row = r0 + wm * 128 + m;
              if constexpr (ATOMIC) atomicAdd(out + (size_t)p.row_token[row] * p.H + n, p.row_w[row] * acc[i][j][r]);
              else out[(size_t)row * p.H + n] = acc[i][j][r];
            }
          }
      }
    }
  }
}

// MODE 0: gate/up + SwiGLU -> h (bf16).  MODE 1: down + combine epilogue.
// GATHER (mode 0): A row r is a[row_token[r]].  ATOMIC (mode 1): fused combine.
template <int MODE, bool GATHER, bool ATOMIC>
__global__ __launch_bounds__(NTHR, 1) void ffn_dma_kernel(TileParams p) {
  __shared__ __attribute__((aligned(1024))) char lds[STAGES][STAGE_BYTES];  // 128 KB
  const int K = MODE == 0 ? p.H : p.I;
  const int Nw = MODE == 0 ? 2 * p.I : p.H;
  const int NT = MODE == 0 ? (p.I + 127) / 128 : (p.H + BN - 1) / BN;
  int e, nt, r0, rows;
  if (!ffn::find_tile<BM>(p, NT, e, nt, r0, rows)) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;
  const int mvalid = rows - wm * 128;
  const int nmb = __builtin_amdgcn_readfirstlane(mvalid <= 0 ? 0 : min(4, (mvalid + 31) >> 5));

  // Sources of this lane's slots: segment s (1 KB) holds tile rows 16s .. 16s+15;
  // slot i of the segment is row 16s + i/4, chunk (i%4) ^ ((row >> 2) & 3).
  DmaSrc src;
  const char *abase = (const char *)p.a;
  const char *bbase = (const char *)p.w + (size_t)e * Nw * K * 2;
#pragma unroll
  for (int u = 0; u < 2; u++) {
    const int row = (2 * wave + u) * 16 + (lane >> 2);
    const int chunk = (lane & 3) ^ ((row >> 2) & 3);
    const int r = r0 + min(row, rows - 1);  // rows past the end repeat the last valid row
    const uint32_t arow = (MODE == 0 && GATHER) ? (uint32_t)p.row_token[r] : (uint32_t)r;
    src.aoff[u] = arow * (uint32_t)K * 2u + (uint32_t)chunk * 16u;
    int wrow;  // columns past the end (I or H a multiple of 64, not of the tile) read a valid row
    if constexpr (MODE == 0) wrow = ((row >> 5) & 1) * p.I + min(nt * 128 + (row >> 6) * 32 + (row & 31), p.I - 1);
    else wrow = min(nt * BN + row, p.H - 1);
    src.boff[u] = (uint32_t)wrow * (uint32_t)K * 2u + (uint32_t)chunk * 16u;
  }

  switch (nmb) {
    case 0: dma_body<MODE, ATOMIC, 0>(p, abase, bbase, src, K, nt, r0, mvalid, wave, lane, wm, wn, lds); break;
    case 1: dma_body<MODE, ATOMIC, 1>(p, abase, bbase, src, K, nt, r0, mvalid, wave, lane, wm, wn, lds); break;
    case 2: dma_body<MODE, ATOMIC, 2>(p, abase, bbase, src, K, nt, r0, mvalid, wave, lane, wm, wn, lds); break;
    case 3: dma_body<MODE, ATOMIC, 3>(p, abase, bbase, src, K, nt, r0, mvalid, wave, lane, wm, wn, lds); break;
    default: dma_body<MODE, ATOMIC, 4>(p, abase, bbase, src, K, nt, r0, mvalid, wave, lane, wm, wn, lds); break;
  }
}

template <int MODE, bool GATHER, bool ATOMIC>
hipError_t launch_d(const TileParams &tp, int grid, hipStream_t s) {
  hipLaunchKernelGGL((ffn_dma_kernel<MODE, GATHER, ATOMIC>), dim3(grid), dim3(NTHR), 0, s, tp);
  return hipGetLastError();
}

}  // namespace

int ffn_dma_bm() { return BM; }

// One or both halves of the bf16-weight large-batch FFN; tp.sched must hold the
// prefix of 256-row tiles.
hipError_t launch_ffn_dma(const TileParams &base, const FfnArgs &a, hipStream_t s) {
  hipError_t err = hipSuccess;
  const long long mt1 = ((long long)a.R_cap + (long long)a.El * (BM - 1)) / BM;
  const long long mt2 = (long long)a.El * ceil_div_i(a.T, BM);
  const long long max_mt = mt1 < mt2 ? mt1 : mt2;
  TileParams tp = base;
  if (a.phase & 1) {
    tp.a = a.a;
    tp.w = a.w_gu;
    tp.out = a.h;
    const int grid = (int)(max_mt * ceil_div_i(a.I, 128));
    err = a.gather ? launch_d<0, true, false>(tp, grid, s) : launch_d<0, false, false>(tp, grid, s);
    if (err != hipSuccess) return err;
  }
  if (a.phase & 2) {
    tp.a = a.h;
    tp.w = a.w_d;
    const bool atomic = a.y != nullptr;
    tp.out = atomic ? (void *)a.y : (void *)a.y_perm;
    const int grid = (int)(max_mt * ceil_div_i(a.H, BN));
    err = atomic ? launch_d<1, false, true>(tp, grid, s) : launch_d<1, false, false>(tp, grid, s);
  }
  return err;
}

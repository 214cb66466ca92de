// Grouped FFN tiles for large batches with bf16 weights: operands move from
// HBM/L2 straight into LDS (global_load_lds, no register staging).
//
// Tile: up to 256 rows of one expert x 256 weight rows, K step 64 (one full
// 128-byte line per row and step).  An expert with c rows is cut into
// m = ceil(c / 256) M tiles of equal size rounded up to 64 rows, so an expert
// of 375 rows runs as two tiles of 192 rows rather than 256 + 119.  Eight
// waves as 2 (M) x 4 (N); each wave owns half the tile rows x 64 weight rows
// as up to 4 x 2 blocks of v_mfma_f32_32x32x16_bf16 (fp32 accumulation).
// Gate/up tiles hold the gate rows and the up rows of the same 128
// intermediate columns, so the SwiGLU epilogue finds G and U of one output in
// the same lane and register.
//
// Pipeline: the weight operand, whose first touch comes from HBM, is fetched
// two K steps ahead through a three-slot ring; the activation rows, mostly L2
// hits, one step ahead through a two-slot ring (2 x 32 KB + 3 x 32 KB = 160 KB
// of LDS, one workgroup per CU).  The loads of the next steps are issued
// between the MFMAs of the current step, two per 16-wide K slice, so no wave
// stalls on a long burst of memory instructions.  Per K step: wait until this
// wave's loads of the step have landed (vmcnt; loads retire in issue order),
// one barrier (everyone's loads have landed and nobody still reads the slots
// about to be refilled), then MFMAs.  The barrier carries no memory fence: a
// fence would drain every load still in flight.
//
// LDS rows are 64 bf16 = eight 16-byte chunks; chunk c of row r sits in slot
// c ^ ((r >> 1) & 7), which keeps the 16 lanes of one LDS cycle on 16 distinct
// 16-byte bank groups when they read one chunk of 16 consecutive rows.  A
// global_load_lds writes the 16 bytes of lane i to slot i of a 1 KB segment
// (8 rows), so every lane fetches the global chunk that belongs to its slot.
//
// Rows past the expert's count are never multiplied: the K loop is
// instantiated for 0..4 active 32-row blocks per wave.
#include "ffn_common.h"

namespace {

using ffn::TileParams;

constexpr int BM = 256, BN = 256, BK = 64, NTHR = 512;
constexpr int A_BYTES = BM * BK * 2;                  // 32 KB: one activation slot
constexpr int B_BYTES = BN * BK * 2;                  // 32 KB: one weight slot
constexpr int LDS_BYTES = 2 * A_BYTES + 3 * B_BYTES;  // 160 KB

__device__ __forceinline__ int lds_off64(int row, int chunk) { return row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4); }

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ void barrier_no_fence() { asm volatile("s_barrier" ::: "memory"); }

struct DmaSrc {
  uint32_t aoff[4], boff[4];  // byte offsets of this lane's A and B segments at K step 0
  uint32_t bstep;             // bytes from one K step of the weights to the next (row-major or packed)
};

template <int NMB>
__device__ __forceinline__ void dma_kloop(const char *abase, const char *bbase, const DmaSrc &src, int nA, int K,
                                          int wave, int lane, int arow0, int wn, char *lds,
                                          f32x16_t (&acc)[NMB > 0 ? NMB : 1][2]) {
  const int KT = K / BK;
  // A of step kt lives in A slot kt % 2, B of step kt in B slot kt % 3.  Within a step every A load
  // is issued before any B load, so once only the four B loads of step kt+1 are in flight, all of
  // step kt has landed.
  auto loadA = [&](int kt, int u) __attribute__((always_inline)) {
    if (u < nA)
      __builtin_amdgcn_global_load_lds((const void *)(abase + (size_t)kt * BK * 2 + src.aoff[u]),
                                       (lds_void *)(lds + (kt & 1) * A_BYTES + (wave + 8 * u) * 1024), 16, 0, 0);
  };
  auto loadB = [&](int kt, int u) __attribute__((always_inline)) {
    __builtin_amdgcn_global_load_lds((const void *)(bbase + (size_t)kt * src.bstep + src.boff[u]),
                                     (lds_void *)(lds + 2 * A_BYTES + (kt % 3) * B_BYTES + (wave + 8 * u) * 1024), 16, 0,
                                     0);
  };
  auto step = [&](int kt, bool nextA, bool nextB) __attribute__((always_inline)) {
    const char *A = lds + (kt & 1) * A_BYTES, *B = lds + 2 * A_BYTES + (kt % 3) * B_BYTES;
#pragma unroll
    for (int kk = 0; kk < 4; kk++) {
      const int ch = kk * 2 + (lane >> 5);
      bf16x8_t bf[2], af[NMB > 0 ? NMB : 1];
      if constexpr (NMB > 0) {
#pragma unroll
        for (int j = 0; j < 2; j++) bf[j] = *(const bf16x8_t *)(B + lds_off64(wn * 64 + j * 32 + (lane & 31), ch));
#pragma unroll
        for (int i = 0; i < NMB; i++) af[i] = *(const bf16x8_t *)(A + lds_off64(arow0 + i * 32 + (lane & 31), ch));
      }
      if (kk < 2) {
        if (nextA) {
          loadA(kt + 1, 2 * kk);
          loadA(kt + 1, 2 * kk + 1);
        }
      } else if (nextB) {
        loadB(kt + 2, 2 * (kk - 2));
        loadB(kt + 2, 2 * (kk - 2) + 1);
      }
      if constexpr (NMB > 0) {
#pragma unroll
        for (int i = 0; i < NMB; i++)
#pragma unroll
          for (int j = 0; j < 2; j++) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
      }
    }
  };
#pragma unroll
  for (int u = 0; u < 4; u++) loadB(0, u);
#pragma unroll
  for (int u = 0; u < 4; u++) loadA(0, u);
  if (KT > 1) {
#pragma unroll
    for (int u = 0; u < 4; u++) loadB(1, u);
  }
  for (int kt = 0; kt < KT; kt++) {
    if (kt + 1 < KT) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    barrier_no_fence();
    step(kt, kt + 1 < KT, kt + 2 < KT);
  }
}

template <int MODE, bool ATOMIC, int NMB>
__device__ __forceinline__ void dma_body(const TileParams &p, const char *abase, const char *bbase, const DmaSrc &src,
                                         int nA, int K, int nt, int rbase, int mvalid, int wave, int lane, int arow0,
                                         int wn, char *lds) {
  constexpr int NA = NMB > 0 ? NMB : 1;
  f32x16_t acc[NA][2];
#pragma unroll
  for (int i = 0; i < NA; i++)
#pragma unroll
    for (int j = 0; j < 2; j++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[i][j][r] = 0.0f;
  dma_kloop<NMB>(abase, bbase, src, nA, K, wave, lane, arow0, wn, lds, acc);
  if constexpr (NMB > 0) {
    // acc[i][j][r] at lane l is tile row arow0 + i*32 + 8*(r/4) + 4*(l/32) + r%4,
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
            hout[(size_t)(rbase + m) * p.I + col] = f32_to_bf16(silu_fast(acc[i][0][r]) * acc[i][1][r]);
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
              const int row = rbase + m;
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
  __shared__ __attribute__((aligned(1024))) char lds[LDS_BYTES];
  const int K = MODE == 0 ? p.H : p.I;
  const int Nw = MODE == 0 ? 2 * p.I : p.H;
  const int NT = MODE == 0 ? (p.I + 127) / 128 : (p.H + BN - 1) / BN;
  int e, nt, mt, mtiles;
  if (!ffn::locate_tile<BM>(p, NT, e, nt, mt, mtiles)) return;
  // equal split of the expert's rows over its M tiles, rounded up to 64 rows
  const int beg = p.offsets[e], cnt = p.offsets[e + 1] - beg;
  const int trows = __builtin_amdgcn_readfirstlane(min(BM, (((cnt + mtiles - 1) / mtiles) + 63) & ~63));
  const int r0 = beg + mt * trows;
  const int rows = min(trows, min(beg + cnt, p.R_cap) - r0);
  if (rows <= 0) return;
  const int half = trows >> 1;  // rows per M wave, a multiple of 32
  const int nA = trows >> 6;    // A segments (8 rows each) per wave and K step

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;
  const int mvalid = rows - wm * half;
  const int nmb = __builtin_amdgcn_readfirstlane(mvalid <= 0 ? 0 : min(half >> 5, (mvalid + 31) >> 5));

  // Sources of this lane's slots: segment s (1 KB) holds tile rows 8s .. 8s+7; wave w fills
  // segments w + 8u.  Slot i of a segment is row 8s + i/8, chunk (i%8) ^ ((row >> 1) & 7).
  DmaSrc src;
  const char *abase = (const char *)p.a;
  const char *bbase = (const char *)p.w + (size_t)e * Nw * K * 2;
#pragma unroll
  for (int u = 0; u < 4; u++) {
    const int row = (wave + 8 * u) * 8 + (lane >> 3);
    const int chunk = (lane & 7) ^ ((row >> 1) & 7);
    const int r = r0 + min(row, rows - 1);  // rows past the end repeat the last valid row
    const uint32_t arow = (MODE == 0 && GATHER) ? (uint32_t)p.row_token[r] : (uint32_t)r;
    src.aoff[u] = arow * (uint32_t)K * 2u + (uint32_t)chunk * 16u;
    // gate/up tile row 64g + 32h + c: gate (h = 0) or up (h = 1) row of intermediate column
    // nt*128 + 32g + c; columns past the end (I or H a multiple of 64 only) read a valid row
    int wrow;
    if constexpr (MODE == 0) wrow = ((row >> 5) & 1) * p.I + min(nt * 128 + (row >> 6) * 32 + (row & 31), p.I - 1);
    else wrow = min(nt * BN + row, p.H - 1);
    src.boff[u] = (uint32_t)ffn::w_row_off(p.wpacked, (size_t)wrow, K, 2) + (uint32_t)chunk * 16u;
  }
  src.bstep = (uint32_t)ffn::w_chunk_step(p.wpacked, 2);
  const int arow0 = wm * half;
  const int rbase = r0 + arow0;
#define DMA_BODY(n) dma_body<MODE, ATOMIC, n>(p, abase, bbase, src, nA, K, nt, rbase, mvalid, wave, lane, arow0, wn, lds)
  switch (nmb) {
    case 0: DMA_BODY(0); break;
    case 1: DMA_BODY(1); break;
    case 2: DMA_BODY(2); break;
    case 3: DMA_BODY(3); break;
    default: DMA_BODY(4); break;
  }
#undef DMA_BODY
}

template <int MODE, bool GATHER, bool ATOMIC>
hipError_t launch_d(const TileParams &tp, int grid, hipStream_t s) {
  hipLaunchKernelGGL((ffn_dma_kernel<MODE, GATHER, ATOMIC>), dim3(grid), dim3(NTHR), 0, s, tp);
  return hipGetLastError();
}

}  // namespace

int ffn_dma_bm() { return BM; }

// One or both halves of the bf16-weight large-batch FFN.
hipError_t launch_ffn_dma(const TileParams &base, const FfnArgs &a, hipStream_t s) {
  hipError_t err = hipSuccess;
  // worst-case M tiles: sum_e ceil(c_e/BM) <= (R + El*(BM-1))/BM and <= El*ceil(T/BM)
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

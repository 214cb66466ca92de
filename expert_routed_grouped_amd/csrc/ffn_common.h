// Tile bookkeeping shared by the grouped-FFN kernels.
#pragma once
#include "common.h"

namespace ffn {

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

// Locate this workgroup's tile.  Returns false for surplus workgroups.
template <int TBM>
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
  r0 = p.offsets[e] + mt * TBM;
  rows = min(TBM, min(p.offsets[e + 1], p.R_cap) - r0);
  return rows > 0;
}

}  // namespace ffn

// Weight-streaming path for small batches (ffn_stream.hip); M tiles of ffn_stream_bm() rows.
int ffn_stream_bm();
hipError_t launch_ffn_stream(const ffn::TileParams &base, const FfnArgs &a, hipStream_t s);

// Direct-to-LDS pipelined tiles for bf16 weights (ffn_dma.hip); M tiles of ffn_dma_bm() rows.
int ffn_dma_bm();
hipError_t launch_ffn_dma(const ffn::TileParams &base, const FfnArgs &a, hipStream_t s);

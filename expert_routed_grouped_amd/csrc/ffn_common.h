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
  int El, H, I;
  int R_cap;              // rows past R_cap are never touched, whatever the offsets say
  int ksplit;             // weight-streaming kernel: K slices per tile (0 or 1: none)
  float *gu32;            // with ksplit > 1: fp32 G and U partial sums [R_cap, 2I], zeroed beforehand
  int wpacked;            // weights in 32-row x 64-k blocks (moe_pack_weights) instead of row-major
  int T;                  // tokens (rows of x when the gate/up half gathers)
};

// Weight addressing for row-major or packed weights of esz bytes; ``row`` counts over all experts
// of the tensor.  Packed: every 32 rows form K/64 consecutive blocks of 32 x 64 values (4 KB of
// bf16, 2 KB of fp8).  Inside an fp8 block the rows follow each other (64 bytes each).  Inside a
// bf16 block, 16-byte piece c (values 8c .. 8c+7 of the chunk) of block row n sits at byte
// (c % 4) * 1024 + (n + 32 * (c / 4)) * 16: a wave that streams the block in the operand layout
// of v_mfma_f32_32x32x16_bf16 (lane n + 32g takes pieces 4g .. 4g+3 of row n) then reads 1 KB
// contiguously per load, and eight consecutive rows of one piece column are 128 contiguous bytes.

// Byte offset of 16-byte piece c (values 16c/esz .. of the row's first 64-wide K chunk) of ``row``.
__device__ __forceinline__ size_t w_piece_off(int packed, size_t row, int c, int K, int esz) {
  if (!packed) return row * (size_t)K * esz + (size_t)c * 16;
  const size_t blk = (row >> 5) * 32 * (size_t)K * esz;
  if (esz == 2) return blk + (size_t)(c & 3) * 1024 + ((row & 31) + 32 * (size_t)(c >> 2)) * 16;
  return blk + (row & 31) * 64 + (size_t)c * 16;
}
// Byte offset of ``row`` at k = 0 (its piece 0).
__device__ __forceinline__ size_t w_row_off(int packed, size_t row, int K, int esz) {
  return w_piece_off(packed, row, 0, K, esz);
}
// Bytes from one 64-wide K chunk of a row to the next.
__device__ __forceinline__ size_t w_chunk_step(int packed, int esz) { return (size_t)(packed ? 32 * 64 : 64) * esz; }
// Bytes from piece c to piece c + 1 of one lane's 4 (bf16) or 2 (fp8) pieces of a chunk, whose
// first piece is a multiple of their count.
__device__ __forceinline__ size_t w_lane_piece_step(int packed, int esz) { return packed && esz == 2 ? 1024 : 16; }

__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__device__ __forceinline__ int wave_incl_scan_i(int v, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(v, off, 64);
    if (lane >= off) v += o;
  }
  return v;
}

// M tiles of TBM rows that expert i needs (0 for an empty or malformed range).
template <int TBM>
__device__ __forceinline__ int expert_mtiles(const TileParams &p, int i) {
  if (i >= p.El) return 0;
  const int c = p.offsets[i + 1] - p.offsets[i];
  return c > 0 ? (c + TBM - 1) / TBM : 0;
}

// Locate this workgroup's tile straight from the expert offsets (no schedule buffer): expert e
// owns ceil(c_e / TBM) M tiles x NT N tiles, numbered expert-major, then N tile, then M tile.
// Workgroups go round-robin over the 8 XCDs, so workgroup b takes tile number
// (b % 8) * total/8 + b / 8: runs of consecutive tiles -- the M and N tiles of one expert, which
// share operands -- stay on one XCD and its L2.  Every wave computes the same answer.
// Returns false for surplus workgroups.
template <int TBM>
__device__ __forceinline__ bool locate_tile(const TileParams &p, int NT, int &e, int &nt, int &mt, int &mtiles) {
  const int lane = threadIdx.x & 63;
  int total = 0;
  for (int b = 0; b < p.El; b += 64) total += wave_sum_i(expert_mtiles<TBM>(p, b + lane));
  total *= NT;
  const int bid = blockIdx.x;
  if (bid >= total) return false;
  const int xcd = bid & 7, j = bid >> 3, q = total >> 3, rem = total & 7;
  const int L = xcd * q + min(xcd, rem) + j;
  int carry = 0;  // M tiles of the experts before this chunk
  for (int b = 0; b < p.El; b += 64) {
    const int t = expert_mtiles<TBM>(p, b + lane);
    const int incl = wave_incl_scan_i(t, lane);
    const unsigned long long hit = __ballot((carry + incl) * NT > L);
    if (hit) {
      const int l = __ffsll((long long)hit) - 1;
      e = b + l;
      mtiles = __shfl(t, l, 64);
      const int rr = L - (carry + __shfl(incl, l, 64) - mtiles) * NT;
      nt = rr / mtiles;
      mt = rr - nt * mtiles;
      return true;
    }
    carry += __shfl(incl, 63, 64);
  }
  return false;
}

// Tile of TBM consecutive rows of one expert (the last tile of an expert may be short).
template <int TBM>
__device__ __forceinline__ bool find_tile(const TileParams &p, int NT, int &e, int &nt, int &r0, int &rows) {
  int mt, mtiles;
  if (!locate_tile<TBM>(p, NT, e, nt, mt, mtiles)) return false;
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

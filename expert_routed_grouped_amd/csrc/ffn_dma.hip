// Grouped FFN tiles for large batches with bf16 or e4m3 (per-output-channel
// scale) weights: operands move from HBM/L2 straight into LDS (buffer_load ...
// lds, no register staging); e4m3 codes are converted to bf16 exactly after
// each fragment read, and their scales multiply the fp32 sums in the epilogue.
//
// Tile: up to 256 rows of one expert x 256 weight rows, K step 64 (one full
// 128-byte line per row and step).  An expert with c rows is cut into
// m = ceil(c / 256) M tiles of equal size rounded up to 64 rows, so an expert
// of 375 rows runs as two tiles of 192 rows rather than 256 + 119.  Eight
// waves, two per SIMD, as 2 (M) x 4 (N); each wave owns half the tile rows x
// 64 weight rows as up to 4 x 2 blocks of v_mfma_f32_32x32x16_bf16 (fp32
// accumulation).  Gate/up tiles hold the gate rows and the up rows of the same
// 128 intermediate columns, so the SwiGLU epilogue finds G and U of one output
// in the same lane and register.
//
// Pipeline: the weight operand, whose first touch comes from HBM, is fetched
// two K steps ahead through a three-slot ring; the activation rows, mostly L2
// hits, one step ahead through a two-slot ring (2 x 32 KB + 3 x 32 KB = 160 KB
// of LDS, or 2 x 32 KB + 3 x 16 KB of e4m3 codes; one workgroup per CU).  The loads of the next steps are issued
// between the MFMAs of the current step, and the fragments of the next 16-wide
// K slice are read while the MFMAs of the current one run.  Per K step: wait
// until this wave's loads of the step have landed (vmcnt; loads retire in
// issue order), one barrier (everyone's loads have landed and nobody still
// reads the slots about to be refilled), then MFMAs.  The barrier carries no
// memory fence: a fence would drain every load still in flight.
//
// Instruction economy of the K loop (it runs at the chip's power limit, so
// every issued instruction costs MFMA clock): the loads are buffer loads whose
// per-lane byte offset is fixed for the whole tile and whose K advance is one
// scalar offset, and the LDS destination (M0) is scalar arithmetic; the loop is
// unrolled over the lcm of the two ring lengths (6 steps), so every fragment
// read is a precomputed per-lane base plus an immediate offset.  The loop body
// then holds MFMAs, LDS reads, loads and a few scalar instructions only.
//
// LDS rows are 64 bf16 = eight 16-byte chunks; chunk c of row r sits in slot
// c ^ ((r >> 1) & 7), which keeps the 16 lanes of one LDS cycle on 16 distinct
// 16-byte bank groups when they read one chunk of 16 consecutive rows.  A load
// to LDS writes the 16 bytes of lane i to slot i of a 1 KB segment (8 rows), so
// every lane fetches the global chunk that belongs to its slot.  Packed weights
// are copied into LDS in their own block layout (chunk c of block row r at
// (c % 4) * 1024 + (r + 32 (c / 4)) * 16 of a 4 KB block): every load then
// reads 1 KB that is contiguous in memory, and a fragment read is two runs of
// 512 contiguous bytes, free of bank conflicts without a swizzle.
//
// Rows past the expert's count are never multiplied: the K loop is
// instantiated for 0..4 active 32-row blocks per wave.  With bf16 weights the
// fp32 sums of every output run over K in the same order as in a plain
// 16-wide-slice MFMA chain; e4m3 weights use a fixed permutation of each
// 64-wide K step (see dma_kloop).
#include "ffn_common.h"

#include <type_traits>

namespace {

using ffn::TileParams;

constexpr int BM = 256, BN = 256, BK = 64, NWAVE = 8, NTHR = 64 * NWAVE;
constexpr int WN = NWAVE / 2;                         // waves along N (two along M)
constexpr int A_BYTES = BM * BK * 2;                  // 32 KB: one activation slot
constexpr int NB = 8 / WN;                            // 32-row weight blocks per wave
constexpr int A_SEG = BM / 8 / NWAVE;                 // most activation segments per wave and K step

// Weight layouts in global memory and LDS (template argument WL):
//   W_ROW: bf16, row-major; LDS rows of 128 bytes with swizzled 16-byte chunks (as the activations)
//   W_PACK: bf16, packed blocks (moe_pack_weights), copied into LDS unchanged
//   W_FP8: e4m3 codes, row-major or packed (row-major 32 x 64-byte blocks); LDS rows of 64 bytes
//          whose 16-byte pieces are swizzled, converted to bf16 after the LDS read
enum { W_ROW = 0, W_PACK = 1, W_FP8 = 2 };
template <int WL>
struct Wt {
  static constexpr int BYTES = BN * BK * (WL == W_FP8 ? 1 : 2);  // one weight slot: 32 KB, or 16 KB of codes
  static constexpr int SEG = BYTES / 1024 / NWAVE;              // weight segments (1 KB) per wave and K step
  static constexpr int LDS = 2 * A_BYTES + 3 * BYTES;           // 160 KB, or 112 KB
};
constexpr int B_SEG_MAX = Wt<W_ROW>::SEG;

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ void barrier_no_fence() { asm volatile("s_barrier" ::: "memory"); }

struct DmaSrc {
  __amdgpu_buffer_rsrc_t ra, rb;  // buffer resources: activations (whole tensor), this expert's weights
  uint32_t aoff[A_SEG], boff[B_SEG_MAX];  // byte offsets of this lane's A and B segments at K step 0
  uint32_t bstep;                 // bytes from one K step of the weights to the next (row-major or packed)
};

constexpr uint32_t kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format (gfx9 family)

// 8 e4m3 codes (two words) -> 8 bf16 (exact).
__device__ __forceinline__ bf16x8_t codes_to_bf16x8(uint32_t w0, uint32_t w1) {
  const uint2 a = e4m3x4_to_bf16x4(w0), b = e4m3x4_to_bf16x4(w1);
  return __builtin_bit_cast(bf16x8_t, u32x4_t{a.x, a.y, b.x, b.y});
}

// One K step with compile-time ring slots: P = kt % 6 (A slot P % 2, B slot P % 3).  Fragment bases:
// abase[kk] (A, 16-wide slice kk), bbase[slot][kk] (bf16 weights) or bbase[slot][j] (e4m3: the
// 16-byte piece j of this lane's row, which holds its codes of slices 2j and 2j+1).
template <int NMB, int P, int WL>
__device__ __forceinline__ void dma_step(int kt, bool nextA, bool nextB, const DmaSrc &src, int nA, int wave,
                                         const uint32_t (&abase)[4], const uint32_t (&bbase)[3][4], char *lds,
                                         f32x16_t (&acc)[NMB > 0 ? NMB : 1][NB]) {
  constexpr int NA = NMB > 0 ? NMB : 1;
  constexpr int SA = P % 2, SB = P % 3, SA1 = (P + 1) % 2, SB2 = (P + 2) % 3;
  constexpr int BSEG = Wt<WL>::SEG, BROW = WL == W_FP8 ? 2048 : 4096;  // LDS bytes of 32 weight rows
  u32x4_t braw[NB];  // e4m3: the piece of slices kk and kk+1 (kk even)
  auto frags = [&](int kk, bf16x8_t (&af)[NA], bf16x8_t (&bf)[NB]) __attribute__((always_inline)) {
    if constexpr (WL == W_FP8) {
      if ((kk & 1) == 0) {
#pragma unroll
        for (int j = 0; j < NB; j++) braw[j] = *(const u32x4_t *)(lds + bbase[SB][kk >> 1] + j * BROW);
      }
#pragma unroll
      for (int j = 0; j < NB; j++)
        bf[j] = (kk & 1) ? codes_to_bf16x8(braw[j].z, braw[j].w) : codes_to_bf16x8(braw[j].x, braw[j].y);
    } else {
#pragma unroll
      for (int j = 0; j < NB; j++) bf[j] = *(const bf16x8_t *)(lds + bbase[SB][kk] + j * BROW);
    }
#pragma unroll
    for (int i = 0; i < NA; i++) af[i] = *(const bf16x8_t *)(lds + abase[kk] + SA * A_BYTES + i * 4096);
  };
  bf16x8_t af[2][NA], bf[2][NB];
  if constexpr (NMB > 0) frags(0, af[0], bf[0]);
  const uint32_t soA = (uint32_t)(kt + 1) * (BK * 2), soB = (uint32_t)(kt + 2) * src.bstep;
#pragma unroll
  for (int kk = 0; kk < 4; kk++) {
    if constexpr (NMB > 0) {
      if (kk < 3) frags(kk + 1, af[(kk + 1) & 1], bf[(kk + 1) & 1]);
    }
    if (kk < 2) {
      if (nextA) {
#pragma unroll
        for (int v = 0; v < (A_SEG + 1) / 2; v++) {
          const int u = (A_SEG + 1) / 2 * kk + v;
          if (u < nA)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                src.ra, (lds_void *)(lds + SA1 * A_BYTES + (wave + NWAVE * u) * 1024), 16, src.aoff[u], soA, 0, 0);
        }
      }
    } else if (nextB) {
#pragma unroll
      for (int v = 0; v < BSEG / 2; v++) {
        const int u = BSEG / 2 * (kk - 2) + v;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            src.rb, (lds_void *)(lds + 2 * A_BYTES + SB2 * Wt<WL>::BYTES + (wave + NWAVE * u) * 1024), 16,
            src.boff[u], soB, 0, 0);
      }
    }
    if constexpr (NMB > 0) {
#pragma unroll
      for (int i = 0; i < NMB; i++)
#pragma unroll
        for (int j = 0; j < NB; j++)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[kk & 1][i], bf[kk & 1][j], acc[i][j], 0, 0, 0);
    }
  }
}

template <int NMB, int WL>
__device__ __forceinline__ void dma_kloop(const DmaSrc &src, int nA, int K, int wave, int lane, int arow0, int wn,
                                          char *lds, f32x16_t (&acc)[NMB > 0 ? NMB : 1][NB]) {
  const int KT = K / BK;
  constexpr int B_SEG = Wt<WL>::SEG, B_BYTES = Wt<WL>::BYTES;
  // LDS byte offsets of this lane's fragments: row r, 16-byte chunk ch = 2 kk + lane / 32 at slot
  // ch ^ ((r >> 1) & 7); rows of one lane differ by multiples of 32, which leave that XOR alone.
  // Packed bf16 weights keep the global block layout in LDS instead: chunk ch of block row r at
  // (ch % 4) * 1024 + (r + 32 * (ch / 4)) * 16 of its 4 KB block, where the 32 lanes of one
  // fragment row read 512 contiguous bytes.  e4m3 weights: 16-byte piece q of weight row r at
  // r * 64 + (q ^ ((r >> 2) & 3)) * 16 (16 lanes reading one piece of 16 consecutive rows hit 16
  // distinct 16-byte bank groups).  Lane (r, g) reads piece j = 2 (kk / 2) + g for slices kk, kk+1
  // and passes its codes 0-7 in slice kk, 8-15 in slice kk+1, so the A fragment of slice kk is the
  // activation chunk 4 (kk / 2) + 2g + kk % 2 (the same k: a permutation of the contraction that
  // both operands share).
  uint32_t abase[4], bbase[3][4];
  {
    const int r = lane & 31, sw = (r >> 1) & 7, g = lane >> 5;
#pragma unroll
    for (int kk = 0; kk < 4; kk++) {
      const int cha = WL == W_FP8 ? 4 * (kk >> 1) + 2 * g + (kk & 1) : 2 * kk + g;
      abase[kk] = (uint32_t)(arow0 + r) * 128u + (uint32_t)((cha ^ sw) << 4);
      const int ch = 2 * kk + g;
      uint32_t ob;
      if constexpr (WL == W_PACK) ob = (uint32_t)(wn * NB * 4096 + (ch & 3) * 1024 + (r + 32 * (ch >> 2)) * 16);
      else if constexpr (WL == W_ROW) ob = (uint32_t)(wn * NB * 32 + r) * 128u + (uint32_t)((ch ^ sw) << 4);
      else ob = (uint32_t)(wn * NB * 32 + r) * 64u + (uint32_t)((((kk & 1) * 2 + g) ^ ((r >> 2) & 3)) << 4);
#pragma unroll
      for (int s = 0; s < 3; s++) bbase[s][kk] = 2u * A_BYTES + (uint32_t)s * B_BYTES + ob;
    }
  }
  // A of step kt lives in A slot kt % 2, B of step kt in B slot kt % 3.  Within a step every A load
  // is issued before any B load, so once only the B loads of step kt+1 are in flight, all of step
  // kt has landed.
#pragma unroll
  for (int u = 0; u < B_SEG; u++)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src.rb, (lds_void *)(lds + 2 * A_BYTES + (wave + NWAVE * u) * 1024), 16,
                                             src.boff[u], 0, 0, 0);
#pragma unroll
  for (int u = 0; u < A_SEG; u++)
    if (u < nA)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(src.ra, (lds_void *)(lds + (wave + NWAVE * u) * 1024), 16,
                                               src.aoff[u], 0, 0, 0);
  if (KT > 1) {
#pragma unroll
    for (int u = 0; u < B_SEG; u++)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          src.rb, (lds_void *)(lds + 2 * A_BYTES + B_BYTES + (wave + NWAVE * u) * 1024), 16, src.boff[u], src.bstep,
          0, 0);
  }
  auto one = [&](auto PC, int kt) __attribute__((always_inline)) {
    constexpr int P = decltype(PC)::value;
    if (kt < KT) {
      if (kt + 1 < KT) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(B_SEG) : "memory");
      else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      barrier_no_fence();
      dma_step<NMB, P, WL>(kt, kt + 1 < KT, kt + 2 < KT, src, nA, wave, abase, bbase, lds, acc);
    }
  };
  for (int kt = 0; kt < KT; kt += 6) {
    one(std::integral_constant<int, 0>{}, kt);
    one(std::integral_constant<int, 1>{}, kt + 1);
    one(std::integral_constant<int, 2>{}, kt + 2);
    one(std::integral_constant<int, 3>{}, kt + 3);
    one(std::integral_constant<int, 4>{}, kt + 4);
    one(std::integral_constant<int, 5>{}, kt + 5);
  }
}

template <int MODE, bool ATOMIC, int WL, int NMB>
__device__ __forceinline__ void dma_body(const TileParams &p, const DmaSrc &src, int e,
                                         int nA, int K, int nt, int rbase, int mvalid, int wave, int lane, int arow0,
                                         int wn, char *lds) {
  constexpr bool F8 = WL == W_FP8;  // e4m3 weights: per-output-channel scale applied to the sums
  constexpr int NA = NMB > 0 ? NMB : 1;
  f32x16_t acc[NA][NB];
#pragma unroll
  for (int i = 0; i < NA; i++)
#pragma unroll
    for (int j = 0; j < NB; j++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[i][j][r] = 0.0f;
  dma_kloop<NMB, WL>(src, nA, K, wave, lane, arow0, wn, lds, acc);
  if constexpr (NMB > 0) {
    // acc[i][j][r] at lane l is tile row arow0 + i*32 + 8*(r/4) + 4*(l/32) + r%4,
    // weight row wn*128 + j*32 + l%32 of the tile
    if constexpr (MODE == 0) {
      // h through a buffer resource: a per-lane 32-bit byte offset (row rbase + 4*(l/32), this
      // lane's column) plus a wave-uniform offset per accumulator row, so no store needs address
      // arithmetic in vector registers (the whole of h is below 2^31 bytes).  Fully valid row
      // blocks, the common case, skip the row test.
      const __amdgpu_buffer_rsrc_t rh = __builtin_amdgcn_make_buffer_rsrc(
          p.out, (short)0, (int)((size_t)p.R_cap * p.I * 2), kRsrcWord3);
      const int I2 = __builtin_amdgcn_readfirstlane(p.I * 2);
      const int voff0 = ((rbase + 4 * (lane >> 5)) * p.I + nt * 128 + wn * NB * 16 + (lane & 31)) * 2;
      auto put = [&](auto FULL) __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < NB / 2; q++) {  // blocks 2q (gate) and 2q+1 (up) of the same 32 columns
          if (nt * 128 + wn * NB * 16 + q * 32 >= p.I) continue;
          float sg = 1.0f, su = 1.0f;
          if constexpr (F8) {
            const size_t c = (size_t)e * 2 * p.I + nt * 128 + wn * NB * 16 + q * 32 + (lane & 31);
            sg = p.scale[c];
            su = p.scale[c + p.I];
          }
          auto hval = [&](float g, float u) __attribute__((always_inline)) {
            if constexpr (F8) return silu_fast(g * sg) * (u * su);
            else return silu_fast(g) * u;
          };
#pragma unroll
          for (int i = 0; i < NA; i++)
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
              const int d = i * 32 + 8 * (r >> 2) + (r & 3);  // row offset of acc r; r+1 is one row below
              const uint32_t hv = pack_bf16x2(hval(acc[i][2 * q][r], acc[i][2 * q + 1][r]),
                                              hval(acc[i][2 * q][r + 1], acc[i][2 * q + 1][r + 1]));
              const int m = d + 4 * (lane >> 5);
              if (decltype(FULL)::value || m < mvalid)
                __builtin_amdgcn_raw_buffer_store_b16((uint16_t)hv, rh, voff0 + q * 64, d * I2, 0);
              if (decltype(FULL)::value || m + 1 < mvalid)
                __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(hv >> 16), rh, voff0 + q * 64, (d + 1) * I2, 0);
            }
        }
      };
      if (mvalid >= NA * 32) put(std::true_type{});
      else put(std::false_type{});
    } else {
      if constexpr (ATOMIC) {
        float *out = (float *)p.out;
#pragma unroll
        for (int j = 0; j < NB; j++) {
          const int n = nt * BN + wn * NB * 32 + j * 32 + (lane & 31);
          if (n >= p.H) continue;
          const float sc = F8 ? p.scale[(size_t)e * p.H + n] : 1.0f;
#pragma unroll
          for (int i = 0; i < NA; i++)
#pragma unroll
            for (int r = 0; r < 16; r++) {
              const int m = i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
              if (m < mvalid) {
                const int row = rbase + m;
                const float o = F8 ? acc[i][j][r] * sc : acc[i][j][r];
                atomicAdd(out + (size_t)p.row_token[row] * p.H + n, p.row_w[row] * o);
              }
            }
        }
      } else {
        // y_perm through a buffer resource, as h above: the whole of it is below 2^32 bytes
        const __amdgpu_buffer_rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc(
            p.out, (short)0, (int)(uint32_t)((size_t)p.R_cap * p.H * 4), kRsrcWord3);
        const uint32_t H4 = (uint32_t)__builtin_amdgcn_readfirstlane(p.H * 4);
        auto put = [&](auto FULL) __attribute__((always_inline)) {
#pragma unroll
          for (int j = 0; j < NB; j++) {
            const int n = nt * BN + wn * NB * 32 + j * 32 + (lane & 31);
            if (n >= p.H) continue;
            const float sc = F8 ? p.scale[(size_t)e * p.H + n] : 1.0f;
            const uint32_t voff = ((uint32_t)(rbase + 4 * (lane >> 5)) * (uint32_t)p.H + (uint32_t)n) * 4u;
#pragma unroll
            for (int i = 0; i < NA; i++)
#pragma unroll
              for (int r = 0; r < 16; r++) {
                const int d = i * 32 + 8 * (r >> 2) + (r & 3);
                const float o = F8 ? acc[i][j][r] * sc : acc[i][j][r];
                if (decltype(FULL)::value || d + 4 * (lane >> 5) < mvalid)
                  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(o), ry, (int)voff, (int)((uint32_t)d * H4), 0);
              }
          }
        };
        if (mvalid >= NA * 32) put(std::true_type{});
        else put(std::false_type{});
      }
    }
  }
}

// MODE 0: gate/up + SwiGLU -> h (bf16).  MODE 1: down + combine epilogue.
// GATHER (mode 0): A row r is a[row_token[r]].  ATOMIC (mode 1): fused combine.
template <int MODE, bool GATHER, bool ATOMIC, int WL>
__global__ __launch_bounds__(NTHR, 1) __attribute__((amdgpu_waves_per_eu(NWAVE / 4, NWAVE / 4))) void ffn_dma_kernel(
    TileParams p) {
  constexpr int WESZ = WL == W_FP8 ? 1 : 2;  // weight bytes per value
  __shared__ __attribute__((aligned(1024))) char lds[Wt<WL>::LDS];
  const int K = MODE == 0 ? p.H : p.I;
  const int Nw = MODE == 0 ? 2 * p.I : p.H;
  const int NT = MODE == 0 ? (p.I + 127) / 128 : (p.H + BN - 1) / BN;
  int e, nt, mt, mtiles;
  if (!ffn::locate_tile<BM>(p, NT, e, nt, mt, mtiles)) return;
  e = __builtin_amdgcn_readfirstlane(e);  // the same in every lane: keep it scalar
  nt = __builtin_amdgcn_readfirstlane(nt);
  mt = __builtin_amdgcn_readfirstlane(mt);
  mtiles = __builtin_amdgcn_readfirstlane(mtiles);
  // equal split of the expert's rows over its M tiles, rounded up to 64 rows
  const int beg = p.offsets[e], cnt = p.offsets[e + 1] - beg;
  const int trows = __builtin_amdgcn_readfirstlane(min(BM, (((cnt + mtiles - 1) / mtiles) + 63) & ~63));
  const int r0 = beg + mt * trows;
  const int rows = min(trows, min(beg + cnt, p.R_cap) - r0);
  if (rows <= 0) return;
  const int half = trows >> 1;  // rows per M wave, a multiple of 32
  const int nA = trows / (8 * NWAVE);  // A segments (8 rows each) per wave and K step

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int mvalid = rows - wm * half;
  const int nmb = __builtin_amdgcn_readfirstlane(mvalid <= 0 ? 0 : min(half >> 5, (mvalid + 31) >> 5));

  // Sources of this lane's slots: segment s (1 KB) of the activation tile holds tile rows
  // 8s .. 8s+7 (likewise for row-major weights); wave w fills segments w + NWAVE u.  Slot i of such
  // a segment is row 8s + i/8, chunk (i%8) ^ ((row >> 1) & 7).
  DmaSrc src;
  {
    const int arows = (MODE == 0 && GATHER) ? p.T : p.R_cap;  // rows of the activation tensor
    src.ra = __builtin_amdgcn_make_buffer_rsrc((void *)p.a, (short)0, (int)((size_t)arows * K * 2), kRsrcWord3);
    src.rb = __builtin_amdgcn_make_buffer_rsrc((void *)((const char *)p.w + (size_t)e * Nw * K * WESZ), (short)0,
                                               (int)((size_t)Nw * K * WESZ), kRsrcWord3);
  }
#pragma unroll
  for (int u = 0; u < A_SEG; u++) {
    const int row = (wave + NWAVE * u) * 8 + (lane >> 3);
    const int chunk = (lane & 7) ^ ((row >> 1) & 7);
    const int r = r0 + min(row, rows - 1);  // rows past the end repeat the last valid row
    const uint32_t arow = (MODE == 0 && GATHER) ? (uint32_t)p.row_token[r] : (uint32_t)r;
    src.aoff[u] = arow * (uint32_t)K * 2u + (uint32_t)chunk * 16u;
  }
#pragma unroll
  for (int u = 0; u < Wt<WL>::SEG; u++) {
    // row-major bf16 weights: the segment's rows and swizzled chunks as for A.  Packed bf16: segment
    // s is chunk column s % 4 of 32-row block s / 4 (slot i: block row i % 32, chunk s % 4 + 4 (i / 32)),
    // 1 KB that lie contiguously in the packed tensor too.  e4m3: segment s holds rows 16s .. 16s+15
    // (slot i: row 16s + i/4, piece (i%4) ^ ((row >> 2) & 3)), 1 KB contiguous in a packed block.
    const int sg = wave + NWAVE * u;
    int row, piece;
    if constexpr (WL == W_PACK) {
      row = (sg >> 2) * 32 + (lane & 31);
      piece = (sg & 3) + 4 * (lane >> 5);
    } else if constexpr (WL == W_ROW) {
      row = sg * 8 + (lane >> 3);
      piece = (lane & 7) ^ ((row >> 1) & 7);
    } else {
      row = sg * 16 + (lane >> 2);
      piece = (lane & 3) ^ ((row >> 2) & 3);
    }
    // gate/up tile row 64g + 32h + c: gate (h = 0) or up (h = 1) row of intermediate column
    // nt*128 + 32g + c; columns past the end (I or H a multiple of 64 only) read a valid row
    int wrow;
    if constexpr (MODE == 0) wrow = ((row >> 5) & 1) * p.I + min(nt * 128 + (row >> 6) * 32 + (row & 31), p.I - 1);
    else wrow = min(nt * BN + row, p.H - 1);
    const int packed = WL == W_PACK ? 1 : (WL == W_ROW ? 0 : p.wpacked);
    src.boff[u] = (uint32_t)ffn::w_piece_off(packed, (size_t)wrow, piece, K, WESZ);
  }
  src.bstep = (uint32_t)ffn::w_chunk_step(WL == W_PACK ? 1 : (WL == W_ROW ? 0 : p.wpacked), WESZ);
  const int arow0 = wm * half;
  const int rbase = r0 + arow0;
#define DMA_BODY(n) dma_body<MODE, ATOMIC, WL, n>(p, src, e, nA, K, nt, rbase, mvalid, wave, lane, arow0, wn, lds)
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
hipError_t launch_d(const TileParams &tp, bool fp8, int grid, hipStream_t s) {
  if (fp8) hipLaunchKernelGGL((ffn_dma_kernel<MODE, GATHER, ATOMIC, W_FP8>), dim3(grid), dim3(NTHR), 0, s, tp);
  else if (tp.wpacked)
    hipLaunchKernelGGL((ffn_dma_kernel<MODE, GATHER, ATOMIC, W_PACK>), dim3(grid), dim3(NTHR), 0, s, tp);
  else hipLaunchKernelGGL((ffn_dma_kernel<MODE, GATHER, ATOMIC, W_ROW>), dim3(grid), dim3(NTHR), 0, s, tp);
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
  tp.T = a.T;
  const bool fp8 = a.w_dt == 2;
  if (a.phase & 1) {
    tp.a = a.a;
    tp.w = a.w_gu;
    tp.scale = a.s_gu;
    tp.out = a.h;
    const int grid = (int)(max_mt * ceil_div_i(a.I, 128));
    err = a.gather ? launch_d<0, true, false>(tp, fp8, grid, s) : launch_d<0, false, false>(tp, fp8, grid, s);
    if (err != hipSuccess) return err;
  }
  if (a.phase & 2) {
    tp.a = a.h;
    tp.w = a.w_d;
    tp.scale = a.s_d;
    const bool atomic = a.y != nullptr;
    tp.out = atomic ? (void *)a.y : (void *)a.y_perm;
    const int grid = (int)(max_mt * ceil_div_i(a.H, BN));
    err = atomic ? launch_d<1, false, true>(tp, fp8, grid, s) : launch_d<1, false, false>(tp, fp8, grid, s);
  }
  return err;
}

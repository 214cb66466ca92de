// W8A8 MXFP8 grouped FFN (moe_grouped_ffn_mx) for gfx950.
//
// Tiling as in the bf16 direct-to-LDS kernel (ffn_dma.hip), with at most 192 rows
// of one expert per tile (equal M tiles per expert, rounded to 64 rows; the fp8
// operand fragments are twice as wide, so 4 x 2 accumulator blocks would spill) x 256 weight rows,
// eight waves as 2 (M) x 4 (N), operands moved HBM/L2 -> LDS by buffer loads to
// LDS with load issue spread over the MFMAs.  The K step is 128 E4M3 values (one
// full 128-byte line per row) plus the four E8M0 scale bytes of each row, and
// the product is v_mfma_scale_f32_32x32x64_f8f6f4: 64 k per instruction with
// the block scales applied inside the matrix core.
//
// Operand layout of that instruction (measured on MI355X): lane l holds row (or
// column) l % 32; with h = l / 32, its bytes 0-15 are k = 16h .. 16h+15 and
// bytes 16-31 are k = 32+16h .. 32+16h+15, so lanes of half h supply the scale
// of the 32-wide block h of the 64 k.  Each lane therefore reads two 16-byte
// chunks of its row per 64 k and passes the row's scale dword shifted by 8h,
// with the byte selector picking block 2*kk of the K step.
//
// LDS: the activation operand of a K step (192 x 128 B) sits in a two-slot ring
// and is fetched one step ahead; the weight operand (256 x 128 B) together with
// the scale dwords of both operands sits in a three-slot ring and is fetched two
// steps ahead (2 x 24 KB + 3 x 34 KB = 150 KB, one workgroup per CU).  When K is
// a multiple of 512 the scales instead move four K steps at a time, 16 bytes per
// lane, into a two-group ring of their own (2 x 24 KB + 3 x 32 KB + 2 x 8 KB =
// 160 KB): a scale load touches one line per lane whatever its size, so this
// cuts the L2 requests of the scales by four.  Every
// wave issues the same loads every step (past the last K step they refetch it
// into slots nobody reads again), so the loop has no branches and the wait at
// the top of a step is a fixed count: everything but this wave's newest loads
// (the weights of the next step, with their scale dwords or a scale group) has
// landed.  One barrier per step.  Chunk c of LDS row r sits in slot
// c ^ ((r >> 1) & 7); wave w's 256-byte scale segment holds the A scales of
// tile rows 32w .. 32w+31, then the B scales of weight rows 32w .. 32w+31.
//
// As in the bf16 kernel the K loop carries no address arithmetic: the code
// loads are buffer loads (per-lane offsets fixed for the tile, the K advance a
// scalar offset, the LDS destination scalar), the loop is unrolled over the
// 6-step period of the two rings so that every fragment and scale read is a
// precomputed per-lane LDS base plus an immediate; only the per-row scale dword
// (one per lane and step) is still a vector-addressed load.
//
// Gate/up epilogue: h = silu(G) * U in fp32, quantised per row in blocks of 32
// intermediate columns (a wave's 32 columns are one block) into MXFP8 codes and
// scales.  Down epilogue: fp32 per-row outputs or the fused atomic combine.
#include "ffn_common.h"
#include "mx_common.h"
#include <type_traits>

namespace {

using ffn::TileParams;

constexpr int BM = 192, BN = 256, BK = 128, NTHR = 512;
constexpr int A_BYTES = BM * BK;                 // 24 KB: one activation slot
constexpr int S_BYTES = NTHR / 64 * 256;         // 2 KB: scale dwords of 8 x 32 A rows and 8 x 32 B rows
constexpr int OFF_B = 2 * A_BYTES;
constexpr int SGRP = NTHR / 64 * 64 * 16;        // 8 KB: the scales of four K steps, 16 bytes per lane
// Two scale schemes (template argument S4):
//   per step: each lane's row scale dword of the step rides in the weight slot (three-slot ring);
//   S4 (K a multiple of 512, scale rows 16-byte aligned): each lane loads its row's scales of four
//      K steps (16 bytes) every four steps into a two-group ring of its own, a quarter of the
//      scale requests (every lane's row is a different line, so each scale load costs 64 L2
//      requests however few bytes it moves).
template <bool S4>
struct Lay {
  static constexpr int BSLOT = BN * BK + (S4 ? 0 : S_BYTES);  // one weight (+ scales) slot: 32 or 34 KB
  static constexpr int OFF_S = OFF_B + 3 * BSLOT;               // S4: the scale groups
  static constexpr int BYTES = OFF_S + (S4 ? 2 * SGRP : 0);     // 160 or 150 KB
  static_assert(BYTES <= 160 * 1024, "fits the LDS of one CU");
};
static_assert(NTHR / 64 * 32 >= BM && NTHR / 64 * 32 >= BN, "scale segments cover every tile row");

typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ void barrier_no_fence() { asm volatile("s_barrier" ::: "memory"); }

struct MxParams {
  TileParams tp;               // offsets, row_token, row_w, El, H, I, R_cap; tp.a / tp.w / tp.out: codes
  const uint8_t *a_scales;     // [rows, K/32]
  const uint8_t *w_scales;     // [El, Nw, K/32]
  uint8_t *out_scales;         // gate/up: h scales [R_cap, I/32]
};

struct Src {
  __amdgpu_buffer_rsrc_t ra, rb;      // activation codes, this expert's weight codes
  const uint8_t *sptr;                // this lane's scale row: A row (lanes < 32) or B row
  uint32_t aoff[3], boff[4];          // byte offsets of this lane's A / B segment chunks at K step 0
  uint32_t bstep;                     // bytes from one K step of the weight codes to the next (row-major or packed)
};

constexpr uint32_t kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format (gfx9 family)

// One K step with compile-time ring slots: P = kt % 6 (A slot P % 2, B slot P % 3).  The loads of
// the next steps are issued past the last step too (their source step clamped to the last one, into
// slots nobody reads again), so every step issues the same loads and the waits are fixed counts.
template <int NMB, int P, bool S4>
__device__ __forceinline__ void mx_step(int kt, int KT, const Src &src, int wave, const uint32_t (&abase)[4],
                                        const uint32_t (&bbase)[3][4], uint32_t sabase, const uint32_t (&sbbase)[3],
                                        int h, char *lds, f32x16_t (&acc)[NMB > 0 ? NMB : 1][2]) {
  constexpr int NA = NMB > 0 ? NMB : 1;
  constexpr int SA = P % 2, SB = P % 3, SA1 = (P + 1) % 2, SB2 = (P + 2) % 3;
  constexpr int BS = Lay<S4>::BSLOT;
  uint32_t sa[NA], sb[2];
  if constexpr (NMB > 0) {
    if constexpr (S4) {  // group kt / 4 in ring entry (kt / 4) % 2, dword kt % 4 of each lane's 16 bytes
      const uint32_t so = (uint32_t)(((kt >> 2) & 1) * SGRP + (kt & 3) * 4);
#pragma unroll
      for (int j = 0; j < 2; j++) sb[j] = *(const uint32_t *)(lds + sbbase[0] + so + j * 1024) >> (8 * h);
#pragma unroll
      for (int i = 0; i < NMB; i++) sa[i] = *(const uint32_t *)(lds + sabase + so + i * 1024) >> (8 * h);
    } else {
#pragma unroll
      for (int j = 0; j < 2; j++) sb[j] = *(const uint32_t *)(lds + sbbase[SB] + j * 256) >> (8 * h);
#pragma unroll
      for (int i = 0; i < NMB; i++) sa[i] = *(const uint32_t *)(lds + sabase + SB * BS + i * 256) >> (8 * h);
    }
  }
  const uint32_t soA = (uint32_t)min(kt + 1, KT - 1) * BK, soB = (uint32_t)min(kt + 2, KT - 1) * src.bstep;
  const int ktS = min(kt + 2, KT - 1);
  // one 64-k half of the K step; KK is a compile-time constant (the scale byte selector must be)
  auto half_step = [&](auto KKC) __attribute__((always_inline)) {
    constexpr int kk = decltype(KKC)::value;
    v8i_t bf[2], af[NA];
    if constexpr (NMB > 0) {
      auto frag = [&](uint32_t lo_off, uint32_t hi_off) __attribute__((always_inline)) {
        const u32x4_t lo = *(const u32x4_t *)(lds + lo_off);
        const u32x4_t hi = *(const u32x4_t *)(lds + hi_off);
        v8i_t v;
        v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w; v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
        return v;
      };
#pragma unroll
      for (int j = 0; j < 2; j++) bf[j] = frag(bbase[SB][2 * kk] + j * 4096, bbase[SB][2 * kk + 1] + j * 4096);
#pragma unroll
      for (int i = 0; i < NMB; i++)
        af[i] = frag(abase[2 * kk] + SA * A_BYTES + i * 4096, abase[2 * kk + 1] + SA * A_BYTES + i * 4096);
    }
    if constexpr (kk == 0) {
#pragma unroll
      for (int u = 0; u < 3; u++)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(src.ra, (lds_void *)(lds + SA1 * A_BYTES + (wave + 8 * u) * 1024),
                                                 16, src.aoff[u], soA, 0, 0);
    } else {
#pragma unroll
      for (int u = 0; u < 4; u++)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            src.rb, (lds_void *)(lds + OFF_B + SB2 * BS + (wave + 8 * u) * 1024), 16, src.boff[u], soB, 0, 0);
      if constexpr (S4) {
        if ((kt & 3) == 2) {  // the scales of steps kt+2 .. kt+5 (the last group again past the end)
          const int g = min((kt + 2) >> 2, (KT >> 2) - 1);
          __builtin_amdgcn_global_load_lds((const void *)(src.sptr + (size_t)g * 16),
                                           (lds_void *)(lds + Lay<S4>::OFF_S + (((kt + 2) >> 2) & 1) * SGRP + wave * 1024),
                                           16, 0, 0);
        }
      } else {
        __builtin_amdgcn_global_load_lds((const void *)(src.sptr + (size_t)ktS * 4),
                                         (lds_void *)(lds + OFF_B + SB2 * BS + BN * BK + wave * 256), 4, 0, 0);
      }
    }
    if constexpr (NMB > 0) {
#pragma unroll
      for (int i = 0; i < NMB; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[i], bf[j], acc[i][j], 0, 0, 2 * kk, sa[i],
                                                                      2 * kk, sb[j]);
    }
  };
  half_step(std::integral_constant<int, 0>{});
  half_step(std::integral_constant<int, 1>{});
}

template <int NMB, bool S4>
__device__ __forceinline__ void kloop(const Src &src, int K, int wave, int lane, int arow0, int wn, char *lds,
                                      f32x16_t (&acc)[NMB > 0 ? NMB : 1][2]) {
  const int KT = K / BK;
  constexpr int BSLOT = Lay<S4>::BSLOT;
  const int h = lane >> 5, r = lane & 31;
  // LDS byte offsets of this lane's fragment chunks: row r (+ multiples of 32, which leave the
  // swizzle alone), chunks 4 kk + 2 c + h at slot chunk ^ ((r >> 1) & 7), for kk, c in {0, 1}
  uint32_t abase[4], bbase[3][4], sbbase[3];
  {
    const int sw = (r >> 1) & 7;
#pragma unroll
    for (int q = 0; q < 4; q++) {  // q = 2 kk + c
      const uint32_t o = (uint32_t)(((2 * q + h) ^ sw) << 4);
      abase[q] = (uint32_t)(arow0 + r) * 128u + o;
#pragma unroll
      for (int s = 0; s < 3; s++) bbase[s][q] = OFF_B + (uint32_t)s * BSLOT + (uint32_t)(wn * 64 + r) * 128u + o;
    }
#pragma unroll
    for (int s = 0; s < 3; s++)
      sbbase[s] = S4 ? Lay<S4>::OFF_S + (uint32_t)(wn * 2) * 1024u + (32u + r) * 16u
                     : OFF_B + (uint32_t)s * BSLOT + BN * BK + (uint32_t)(wn * 2) * 256u + 128u + r * 4u;
  }
  // A scales of tile row arow0 + 32 i + r: segment (arow0 >> 5) + i of the slot's scale area (S4: of
  // the scale group, 16 bytes per lane)
  const uint32_t sabase = S4 ? Lay<S4>::OFF_S + (uint32_t)(arow0 >> 5) * 1024u + r * 16u
                             : OFF_B + BN * BK + (uint32_t)(arow0 >> 5) * 256u + r * 4u;
  // prologue: weights and scales of steps 0 and 1 (S4: the scales of steps 0 .. 3), activations of step 0
#pragma unroll
  for (int u = 0; u < 4; u++)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src.rb, (lds_void *)(lds + OFF_B + (wave + 8 * u) * 1024), 16,
                                             src.boff[u], 0, 0, 0);
  if constexpr (S4)
    __builtin_amdgcn_global_load_lds((const void *)src.sptr, (lds_void *)(lds + Lay<S4>::OFF_S + wave * 1024), 16, 0, 0);
  else
    __builtin_amdgcn_global_load_lds((const void *)src.sptr, (lds_void *)(lds + OFF_B + BN * BK + wave * 256), 4, 0, 0);
#pragma unroll
  for (int u = 0; u < 3; u++)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src.ra, (lds_void *)(lds + (wave + 8 * u) * 1024), 16, src.aoff[u], 0, 0,
                                             0);
  const uint32_t so1 = (uint32_t)min(1, KT - 1);
#pragma unroll
  for (int u = 0; u < 4; u++)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src.rb, (lds_void *)(lds + OFF_B + BSLOT + (wave + 8 * u) * 1024), 16,
                                             src.boff[u], so1 * src.bstep, 0, 0);
  if constexpr (!S4)
    __builtin_amdgcn_global_load_lds((const void *)(src.sptr + (size_t)so1 * 4),
                                     (lds_void *)(lds + OFF_B + BSLOT + BN * BK + wave * 256), 4, 0, 0);
  // this wave's newest loads are the weights of step kt + 1 with their scale dwords (five loads),
  // or with S4 the weights of step kt + 1 (four loads) and, at kt % 4 == 3, the scale group issued
  // after them; all older ones, among them everything step kt reads, have landed once no more than
  // those are in flight
  auto one = [&](auto PC, int kt) __attribute__((always_inline)) {
    constexpr int P = decltype(PC)::value;
    if (kt < KT) {
      if constexpr (S4) {
        if ((kt & 3) == 3) asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
        else asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
      } else {
        asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
      }
      barrier_no_fence();
      mx_step<NMB, P, S4>(kt, KT, src, wave, abase, bbase, sabase, sbbase, h, lds, acc);
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
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

template <int MODE, bool ATOMIC, bool S4, int NMB>
__device__ __forceinline__ void body(const MxParams &mp, const Src &src, int K,
                                     int nt, int rbase, int mvalid, int wave, int lane, int arow0, int wn, char *lds) {
  const TileParams &p = mp.tp;
  constexpr int NA = NMB > 0 ? NMB : 1;
  f32x16_t acc[NA][2];
#pragma unroll
  for (int i = 0; i < NA; i++)
#pragma unroll
    for (int j = 0; j < 2; j++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[i][j][r] = 0.0f;
  kloop<NMB, S4>(src, K, wave, lane, arow0, wn, lds, acc);
  // gate/up: the epilogue stages h in LDS once every wave is past its last operand read (every
  // wave runs the same K steps, so every wave reaches this barrier)
  if constexpr (MODE == 0) __syncthreads();
  if constexpr (NMB > 0) {
    // acc[i][j][r] at lane l is tile row arow0 + i*32 + 8*(r/4) + 4*(l/32) + r%4,
    // weight row wn*64 + j*32 + l%32 of the tile
    if constexpr (MODE == 0) {
      // h = silu(G) U (fp32) goes through this wave's part of the LDS, transposed so that a lane owns
      // whole rows of the wave's 32 intermediate columns, which are exactly one MX block: the lane
      // takes the block maximum over its own 32 values, encodes them four to a dword and stores its
      // 32 codes and the scale byte (no cross-lane reduction, no byte stores).  Staged rows are 36
      // floats apart: 16-byte aligned, and 16 lanes reading the same 16 bytes of 16 rows hit 16
      // distinct groups of banks.
      constexpr int LS = 36;
      float *st = (float *)(lds + wave * (BM / 2) * LS * 4);
#pragma unroll
      for (int i = 0; i < NA; i++)
#pragma unroll
        for (int r = 0; r < 16; r++) {
          const int m = i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          st[m * LS + (lane & 31)] = silu_fast(acc[i][0][r]) * acc[i][1][r];
        }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's rows are staged (LDS is in order per wave)
      const int colbase = nt * 128 + wn * 32;  // first intermediate column of the block; I % 128 == 0
      const int ib = p.I / 32;
      uint8_t *hq = (uint8_t *)p.out;
#pragma unroll
      for (int m0 = 0; m0 < NA * 32; m0 += 64) {
        const int m = m0 + lane;
        if (m < NA * 32 && m < mvalid) {
          f32x4_t v[8];
#pragma unroll
          for (int q = 0; q < 8; q++) v[q] = *(const f32x4_t *)(st + m * LS + 4 * q);
          float amax = 0.0f;
#pragma unroll
          for (int q = 0; q < 8; q++)
#pragma unroll
            for (int c = 0; c < 4; c++) amax = fmaxf(amax, fabsf(v[q][c]));
          const uint32_t sc = mx_scale_of(amax);
          const int ex = 127 - (int)sc;
          u32x4_t w[2];
#pragma unroll
          for (int q = 0; q < 8; q++) {
            const float c0 = fminf(fmaxf(ldexpf(v[q][0], ex), -448.0f), 448.0f);
            const float c1 = fminf(fmaxf(ldexpf(v[q][1], ex), -448.0f), 448.0f);
            const float c2 = fminf(fmaxf(ldexpf(v[q][2], ex), -448.0f), 448.0f);
            const float c3 = fminf(fmaxf(ldexpf(v[q][3], ex), -448.0f), 448.0f);
            const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(c0, c1, 0, false);
            w[q >> 2][q & 3] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c2, c3, lo, true);
          }
          const size_t row = (size_t)(rbase + m);
          *(u32x4_t *)(hq + row * p.I + colbase) = w[0];
          *(u32x4_t *)(hq + row * p.I + colbase + 16) = w[1];
          mp.out_scales[row * ib + colbase / 32] = (uint8_t)sc;
        }
      }
    } else if constexpr (ATOMIC) {
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
              atomicAdd(out + (size_t)p.row_token[row] * p.H + n, p.row_w[row] * acc[i][j][r]);
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
        for (int j = 0; j < 2; j++) {
          const int n = nt * BN + wn * 64 + j * 32 + (lane & 31);
          if (n >= p.H) continue;
          const uint32_t voff = ((uint32_t)(rbase + 4 * (lane >> 5)) * (uint32_t)p.H + (uint32_t)n) * 4u;
#pragma unroll
          for (int i = 0; i < NA; i++)
#pragma unroll
            for (int r = 0; r < 16; r++) {
              const int d = i * 32 + 8 * (r >> 2) + (r & 3);
              if (decltype(FULL)::value || d + 4 * (lane >> 5) < mvalid)
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[i][j][r]), ry, (int)voff,
                                                      (int)((uint32_t)d * H4), 0);
            }
        }
      };
      if (mvalid >= NA * 32) put(std::true_type{});
      else put(std::false_type{});
    }
  }
}

// MODE 0: gate/up + SwiGLU -> h (MXFP8).  MODE 1: down + combine epilogue.
// GATHER (mode 0): A row r is a[row_token[r]].  ATOMIC (mode 1): fused combine.
template <int MODE, bool GATHER, bool ATOMIC, bool S4>
__global__ __launch_bounds__(NTHR, 1) void ffn_mx_kernel(MxParams mp) {
  __shared__ __attribute__((aligned(1024))) char lds[Lay<S4>::BYTES];
  const TileParams &p = mp.tp;
  const int K = MODE == 0 ? p.H : p.I;
  const int Nw = MODE == 0 ? 2 * p.I : p.H;
  const int NT = MODE == 0 ? p.I / 128 : (p.H + BN - 1) / BN;
  int e, nt, mt, mtiles;
  if (!ffn::locate_tile<BM>(p, NT, e, nt, mt, mtiles)) return;
  e = __builtin_amdgcn_readfirstlane(e);  // the same in every lane: keep it scalar
  nt = __builtin_amdgcn_readfirstlane(nt);
  mt = __builtin_amdgcn_readfirstlane(mt);
  mtiles = __builtin_amdgcn_readfirstlane(mtiles);
  const int beg = p.offsets[e], cnt = p.offsets[e + 1] - beg;
  const int trows = __builtin_amdgcn_readfirstlane(min(BM, (((cnt + mtiles - 1) / mtiles) + 63) & ~63));
  const int r0 = beg + mt * trows;
  const int rows = min(trows, min(beg + cnt, p.R_cap) - r0);
  if (rows <= 0) return;
  const int half = trows >> 1;

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int mvalid = rows - wm * half;
  const int nmb = __builtin_amdgcn_readfirstlane(mvalid <= 0 ? 0 : min(half >> 5, (mvalid + 31) >> 5));

  const int kb = K / 32;  // scale bytes per row
  auto a_row = [&](int row) -> uint32_t {  // source row of tile row ``row`` (rows past the end repeat the last)
    const int r = r0 + min(row, rows - 1);
    return (MODE == 0 && GATHER) ? (uint32_t)p.row_token[r] : (uint32_t)r;
  };
  auto w_row = [&](int row) -> int {  // weight row of tile row ``row``
    if constexpr (MODE == 0) return ((row >> 5) & 1) * p.I + nt * 128 + (row >> 6) * 32 + (row & 31);
    else return min(nt * BN + row, p.H - 1);
  };
  Src src;
  const int arows = (MODE == 0 && GATHER) ? p.T : p.R_cap;  // rows of the activation tensor
  src.ra = __builtin_amdgcn_make_buffer_rsrc((void *)p.a, (short)0, (int)((size_t)arows * K), kRsrcWord3);
  src.rb = __builtin_amdgcn_make_buffer_rsrc((void *)((const char *)p.w + (size_t)e * Nw * K), (short)0,
                                             (int)((size_t)Nw * K), kRsrcWord3);
  const uint8_t *asb = mp.a_scales;
  const uint8_t *bsb = mp.w_scales + (size_t)e * Nw * kb;
#pragma unroll
  for (int u = 0; u < 4; u++) {
    const int row = (wave + 8 * u) * 8 + (lane >> 3);
    const int chunk = (lane & 7) ^ ((row >> 1) & 7);
    if (u < 3) src.aoff[u] = a_row(row) * (uint32_t)K + (uint32_t)chunk * 16u;
    // 16-byte chunk c of a 128-value step: row-major at 16c; packed in the 64-value chunk c / 4
    // of the row's 32-row block, at 16 (c % 4) inside its 64-byte piece
    const uint32_t wr = (uint32_t)w_row(row);
    src.boff[u] = p.wpacked ? (wr >> 5) * 32u * (uint32_t)K + (wr & 31u) * 64u + (uint32_t)(chunk >> 2) * 2048u +
                                  (uint32_t)(chunk & 3) * 16u
                            : wr * (uint32_t)K + (uint32_t)chunk * 16u;
  }
  src.bstep = p.wpacked ? 2u * 2048u : (uint32_t)BK;
  {
    const int row = wave * 32 + (lane & 31);
    src.sptr = lane < 32 ? asb + (size_t)a_row(row) * kb : bsb + (size_t)w_row(row) * kb;
  }
  const int arow0 = wm * half;
  const int rbase = r0 + arow0;
#define MX_BODY(n) body<MODE, ATOMIC, S4, n>(mp, src, K, nt, rbase, mvalid, wave, lane, arow0, wn, lds)
  switch (nmb) {
    case 0: MX_BODY(0); break;
    case 1: MX_BODY(1); break;
    case 2: MX_BODY(2); break;
    default: MX_BODY(3); break;
  }
#undef MX_BODY
}

template <int MODE, bool GATHER, bool ATOMIC>
hipError_t launch_m(const MxParams &mp, int grid, hipStream_t s) {
  // S4: K a multiple of 512 (whole four-step scale groups) and every scale row 16-byte aligned
  const int K = MODE == 0 ? mp.tp.H : mp.tp.I;
  const bool s4 = K % 512 == 0 && ((uintptr_t)mp.a_scales & 15) == 0 && ((uintptr_t)mp.w_scales & 15) == 0;
  if (s4) hipLaunchKernelGGL((ffn_mx_kernel<MODE, GATHER, ATOMIC, true>), dim3(grid), dim3(NTHR), 0, s, mp);
  else hipLaunchKernelGGL((ffn_mx_kernel<MODE, GATHER, ATOMIC, false>), dim3(grid), dim3(NTHR), 0, s, mp);
  return hipGetLastError();
}

}  // namespace

size_t ffn_mx_h_bytes(int R_cap, int I) { return align_up((size_t)R_cap * (size_t)I, 256); }

hipError_t launch_ffn_mx(const FfnMxArgs &a, hipStream_t s) {
  if (a.R_cap == 0 || a.T == 0) return hipSuccess;
  // few rows per expert on average: stream the weights (HBM bound), as for bf16 weights
  if (a.kernel == 1 || (a.kernel == 0 && (long long)a.R_cap <= 48LL * a.El)) return launch_ffn_mx_stream(a, s);
  hipError_t err = hipSuccess;
  const long long mt1 = ((long long)a.R_cap + (long long)a.El * (BM - 1)) / BM;
  const long long mt2 = (long long)a.El * ceil_div_i(a.T, BM);
  const long long max_mt = mt1 < mt2 ? mt1 : mt2;
  uint8_t *hq = (uint8_t *)a.ws;
  uint8_t *hs = hq + ffn_mx_h_bytes(a.R_cap, a.I);
  MxParams mp{};
  mp.tp.offsets = a.offsets;
  mp.tp.row_token = a.row_token;
  mp.tp.row_w = a.row_w;
  mp.tp.El = a.El;
  mp.tp.H = a.H;
  mp.tp.I = a.I;
  mp.tp.R_cap = a.R_cap;
  mp.tp.wpacked = a.wpacked;
  mp.tp.T = a.T;
  if (a.phase & 1) {
    MxParams m = mp;
    m.tp.a = a.a;
    m.a_scales = a.a_s;
    m.tp.w = a.wgu;
    m.w_scales = a.wgu_s;
    m.tp.out = hq;
    m.out_scales = hs;
    const int grid = (int)(max_mt * (a.I / 128));
    err = a.gather ? launch_m<0, true, false>(m, grid, s) : launch_m<0, false, false>(m, grid, s);
    if (err != hipSuccess) return err;
  }
  if (a.phase & 2) {
    MxParams m = mp;
    m.tp.a = hq;
    m.a_scales = hs;
    m.tp.w = a.wd;
    m.w_scales = a.wd_s;
    const bool atomic = a.y != nullptr;
    m.tp.out = atomic ? (void *)a.y : (void *)a.y_perm;
    const int grid = (int)(max_mt * ceil_div_i(a.H, BN));
    err = atomic ? launch_m<1, false, true>(m, grid, s) : launch_m<1, false, false>(m, grid, s);
  }
  return err;
}

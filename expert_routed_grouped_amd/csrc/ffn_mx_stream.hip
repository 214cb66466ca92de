// W8A8 MXFP8 grouped FFN for small batches (decode): weight streaming.
//
// Same plan as the bf16 weight-streaming kernel (ffn_stream.hip): with a few
// rows per expert the layer is bound by reading every active expert's weights
// from HBM once, so there is no LDS and no barrier; each wave owns 32 output
// columns of one expert (32 gate + 32 up rows for the gate/up half, two 32-row
// blocks for the down half) for 32 rows of that expert (64 when the rows per
// expert average more than 16), and streams its weight rows straight into
// registers with two K steps in flight.  MXFP8 halves the weight bytes of bf16
// (E4M3 codes plus one E8M0 scale byte per 32 values).
//
// The product is v_mfma_scale_f32_32x32x64_f8f6f4 (block scales applied inside
// the matrix core).  Its operand layout: lane l holds row l % 32; with
// h = l / 32 its bytes 0-15 are k = 16h .. 16h+15 and bytes 16-31 are
// k = 32+16h .. 32+16h+15 of the 64 k, and the lanes of half h supply the scale
// of the 32-wide block h.  A K step is 128 values (one 128-byte line per row),
// two instructions: lane (n, h) loads the 16-byte pieces h, 2+h, 4+h, 6+h of
// its row's line and the row's four scale bytes (one dword), and passes the
// dword shifted by 8h with the byte selector of the instruction's block pair.
//
// Gate/up epilogue: h = silu(G) * U in fp32, quantised per row in blocks of 32
// intermediate columns (a wave's 32 columns are exactly one block, held by the
// 32 lanes of a half) into MXFP8 codes and scales, with the rule of the
// quantisation kernel.  Down epilogue: fp32 per-row outputs or the fused atomic
// combine.
#include "ffn_common.h"
#include "mx_common.h"
#include <type_traits>

namespace {

using ffn::TileParams;

constexpr int XWAVES = 4;            // waves per block
constexpr int XCOLS = 32 * XWAVES;   // gate/up columns per block (down: twice as many)

typedef int v8i_t __attribute__((ext_vector_type(8)));

struct MxsParams {
  TileParams tp;              // offsets, row_token, row_w, El, H, I, R_cap; tp.a / tp.w / tp.out: codes
  const uint8_t *a_scales;    // [rows, K/32]
  const uint8_t *w_scales;    // [El, Nw, K/32]
  uint8_t *out_scales;        // gate/up: h scales [R_cap, I/32]
};

__device__ __forceinline__ v8i_t frag(const u32x4_t &lo, const u32x4_t &hi) {
  v8i_t v;
  v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w; v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
  return v;
}

// MODE 0: gate/up + SwiGLU -> h (MXFP8).  MODE 1: down + combine epilogue.  XMB: 32-row MFMA
// blocks per M tile (1 keeps the registers of two waves per SIMD; 2 streams the weights once per
// 64 rows of an expert at one wave per SIMD).  S4: K is a multiple of 512 and the scale arrays
// are 16-byte aligned, so each row's scales are read 16 bytes (four K steps) at a time instead of
// one dword per step (a quarter of the scale requests).  WLDS (K <= 4096): the wave first copies
// the scale rows of its 64 weight rows (at most 128 bytes, one line, each) into its own part of
// LDS and reads each step's scale dword there, so every scale line leaves HBM once; read from
// memory step by step, a row's scale line is usually evicted from L2 between two steps.
template <int MODE, int XMB, bool S4, bool WLDS, bool GATHER, bool ATOMIC>
__global__ __launch_bounds__(64 * XWAVES) void ffn_mx_stream_kernel(MxsParams mp) {
  constexpr int XBM = 32 * XMB;  // rows per M tile
  constexpr int WSTRIDE = 33;    // LDS dwords per weight row's scales (K <= 4096, one pad dword)
  __shared__ uint32_t wsl[WLDS ? XWAVES : 1][2][32][WLDS ? WSTRIDE : 1];
  const TileParams &p = mp.tp;
  const int K = MODE == 0 ? p.H : p.I;
  const int Ncols = MODE == 0 ? p.I : p.H;
  const int Nw = MODE == 0 ? 2 * p.I : p.H;
  constexpr int WCOLS = MODE == 0 ? 32 : 64;  // output columns per wave
  const int NT = (Ncols + XWAVES * WCOLS - 1) / (XWAVES * WCOLS);
  int e, nt, r0, rows;
  if (!ffn::find_tile<XBM>(p, NT, e, nt, r0, rows)) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c0 = (nt * XWAVES + wave) * WCOLS;
  if (c0 >= Ncols) return;  // Ncols is a multiple of 128: a wave's columns are all valid or all past the end
  const int n = lane & 31, h = lane >> 5;
  const bool two_m = XMB > 1 && rows > 32;  // wave-uniform
  const int kb = K / 32;         // scale bytes per row (a multiple of 4)

  // this lane's weight rows (gate + up, or two down blocks) and activation rows; activation
  // rows past the end repeat the last valid row (their results are never stored)
  const uint8_t *wrow[2], *wsrow[2], *arow[XMB], *asrow[XMB];
  // codes of one K step (128 values): two 64-wide chunks, cstep bytes apart (64 row-major, 2048
  // in the packed 32-row x 64-value blocks)
  const size_t cstep = ffn::w_chunk_step(p.wpacked, 1);
  {
    const size_t r0w = (size_t)e * Nw + c0 + n;
    const size_t r1w = MODE == 0 ? r0w + p.I : r0w + 32;
    wrow[0] = (const uint8_t *)p.w + ffn::w_row_off(p.wpacked, r0w, K, 1) + 16 * h;
    wrow[1] = (const uint8_t *)p.w + ffn::w_row_off(p.wpacked, r1w, K, 1) + 16 * h;
    wsrow[0] = mp.w_scales + r0w * kb;
    wsrow[1] = mp.w_scales + r1w * kb;
  }
#pragma unroll
  for (int mb = 0; mb < XMB; mb++) {
    const int r = r0 + min(mb * 32 + n, rows - 1);
    const size_t src = (MODE == 0 && GATHER) ? (size_t)p.row_token[r] : (size_t)r;
    arow[mb] = (const uint8_t *)p.a + src * K + 16 * h;
    asrow[mb] = mp.a_scales + src * kb;
  }

  f32x16_t acc[XMB][2];
#pragma unroll
  for (int mb = 0; mb < XMB; mb++)
#pragma unroll
    for (int b = 0; b < 2; b++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[mb][b][r] = 0.0f;

  u32x4_t wq[2][2][4], aq[2][XMB][4];
  // scale dwords: per step (S4 false) in the step's buffer, or (S4) 16 bytes = four steps per
  // row, loaded with the first step of each group into ``nxt`` and moved to ``cur`` when that
  // step is computed
  uint32_t wsc[2][2], asc[2][XMB];
  u32x4_t wnxt[2], anxt[XMB], wcur[2], acur[XMB];
  auto load = [&](int buf, int s) __attribute__((always_inline)) {
    const size_t k0 = (size_t)s * 128, w0 = (size_t)s * 2 * cstep;
#pragma unroll
    for (int b = 0; b < 2; b++) {
#pragma unroll
      for (int q = 0; q < 4; q++) wq[buf][b][q] = *(const u32x4_t *)(wrow[b] + w0 + (q >> 1) * cstep + 32 * (q & 1));
      if constexpr (WLDS) {
        // the weight scales are in LDS
      } else if constexpr (S4) {
        if ((s & 3) == 0) wnxt[b] = *(const u32x4_t *)(wsrow[b] + 4 * s);  // s is uniform
      } else {
        wsc[buf][b] = *(const uint32_t *)(wsrow[b] + 4 * s);
      }
    }
#pragma unroll
    for (int mb = 0; mb < XMB; mb++) {
      if (mb > 0 && !two_m) break;
#pragma unroll
      for (int q = 0; q < 4; q++) aq[buf][mb][q] = *(const u32x4_t *)(arow[mb] + k0 + 32 * q);
      if constexpr (S4) {
        if ((s & 3) == 0) anxt[mb] = *(const u32x4_t *)(asrow[mb] + 4 * s);
      } else {
        asc[buf][mb] = *(const uint32_t *)(asrow[mb] + 4 * s);
      }
    }
  };
  // step s from buffer buf (buf == s % 2)
  auto compute = [&](int buf, int s) __attribute__((always_inline)) {
    uint32_t sb[2], sa[XMB];
    if constexpr (S4) {
      if ((s & 3) == 0) {
        if constexpr (!WLDS) {
#pragma unroll
          for (int b = 0; b < 2; b++) wcur[b] = wnxt[b];
        }
#pragma unroll
        for (int mb = 0; mb < XMB; mb++) acur[mb] = anxt[mb];
      }
      const bool hi2 = (s & 2) != 0;
      auto pick = [&](const u32x4_t &v) {
        return buf == 0 ? (hi2 ? v.z : v.x) : (hi2 ? v.w : v.y);
      };
      if constexpr (!WLDS) {
#pragma unroll
        for (int b = 0; b < 2; b++) sb[b] = pick(wcur[b]) >> (8 * h);
      }
#pragma unroll
      for (int mb = 0; mb < XMB; mb++) sa[mb] = pick(acur[mb]) >> (8 * h);
    } else {
      if constexpr (!WLDS) {
#pragma unroll
        for (int b = 0; b < 2; b++) sb[b] = wsc[buf][b] >> (8 * h);
      }
#pragma unroll
      for (int mb = 0; mb < XMB; mb++) sa[mb] = asc[buf][mb] >> (8 * h);
    }
    if constexpr (WLDS) {
#pragma unroll
      for (int b = 0; b < 2; b++) sb[b] = wsl[wave][b][n][s] >> (8 * h);
    }
    // instruction j: pieces 2j, 2j+1 of the lane's loads, blocks 2j (half 0) and 2j+1 (half 1)
    auto pair = [&](auto JC) __attribute__((always_inline)) {
      constexpr int j = decltype(JC)::value;
      v8i_t bo[2];
#pragma unroll
      for (int b = 0; b < 2; b++) bo[b] = frag(wq[buf][b][2 * j], wq[buf][b][2 * j + 1]);
      const v8i_t a0 = frag(aq[buf][0][2 * j], aq[buf][0][2 * j + 1]);
#pragma unroll
      for (int b = 0; b < 2; b++)
        acc[0][b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a0, bo[b], acc[0][b], 0, 0, 2 * j, sa[0], 2 * j,
                                                                    sb[b]);
      if constexpr (XMB > 1) {
        if (two_m) {
          const v8i_t a1 = frag(aq[buf][XMB - 1][2 * j], aq[buf][XMB - 1][2 * j + 1]);
#pragma unroll
          for (int b = 0; b < 2; b++)
            acc[XMB - 1][b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a1, bo[b], acc[XMB - 1][b], 0, 0, 2 * j,
                                                                              sa[XMB - 1], 2 * j, sb[b]);
        }
      }
    };
    pair(std::integral_constant<int, 0>{});
    pair(std::integral_constant<int, 1>{});
  };
  const int KT = K / 128;  // with S4 a multiple of 4
  load(0, 0);
  if constexpr (WLDS) {
    // lane (n, h) copies its half of the scale dwords of row n of both weight blocks; only this
    // wave reads them, and LDS operations of one wave are done in order, so no barrier is needed
    const int kd = kb / 4, half = (kd + 1) / 2;
    const int i0 = h * half, i1 = min(kd, i0 + half);
#pragma unroll
    for (int b = 0; b < 2; b++)
      for (int i = i0; i < i1; i++) wsl[wave][b][n][i] = *(const uint32_t *)(wsrow[b] + 4 * i);
  }
  int s = 0;
  for (; s + 2 <= KT; s += 2) {
    load(1, s + 1);
    compute(0, s);
    if (s + 2 < KT) load(0, s + 2);
    compute(1, s + 1);
  }
  if (s < KT) compute(0, s);

  // ---- epilogue: acc[mb][b][r] at lane l is row mb*32 + 8*(r/4) + 4*(l/32) + r%4, column c0 + l%32
  const int col = c0 + n;
  if constexpr (MODE == 0) {
    uint8_t *hq = (uint8_t *)p.out;
    const int ib = p.I / 32;
#pragma unroll
    for (int mb = 0; mb < XMB; mb++) {
      if (mb == 1 && !two_m) break;  // wave-uniform: every lane joins the shuffles below
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int m = mb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        const float hv = silu_fast(acc[mb][0][r]) * acc[mb][1][r];
        const uint32_t sc = mx_scale_of(halfwave_amax(hv));
        if (m < rows) {
          const size_t row = (size_t)(r0 + m);
          hq[row * p.I + col] = (uint8_t)e4m3_encode(ldexpf(hv, 127 - (int)sc));
          if (n == 0) mp.out_scales[row * ib + col / 32] = (uint8_t)sc;
        }
      }
    }
  } else {
    float *out = (float *)p.out;
#pragma unroll
    for (int b = 0; b < 2; b++) {
      const int cb = col + 32 * b;
#pragma unroll
      for (int mb = 0; mb < XMB; mb++) {
        if (mb == 1 && !two_m) break;
#pragma unroll
        for (int r = 0; r < 16; r++) {
          const int m = mb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
          if (m < rows) {
            const int row = r0 + m;
            if constexpr (ATOMIC) atomicAdd(out + (size_t)p.row_token[row] * p.H + cb, p.row_w[row] * acc[mb][b][r]);
            else out[(size_t)row * p.H + cb] = acc[mb][b][r];
          }
        }
      }
    }
  }
}

template <int MODE, bool GATHER, bool ATOMIC>
hipError_t launch_xs(const MxsParams &mp, int xmb, long long max_mt, int ntiles, hipStream_t s) {
  const int grid = (int)(max_mt * ntiles);
  const int K = MODE == 0 ? mp.tp.H : mp.tp.I;
  const bool s4 = K % 512 == 0 && (((uintptr_t)mp.a_scales | (uintptr_t)mp.w_scales) & 15u) == 0;
  const bool wl = K <= 4096;  // a row's scale dwords fit the LDS row of ffn_mx_stream_kernel
  dim3 g(grid), b(64 * XWAVES);
#define XS_CASE(XMB, S4, WL)                                                                      \
  if (xmb == XMB && s4 == S4 && wl == WL) {                                                      \
    hipLaunchKernelGGL((ffn_mx_stream_kernel<MODE, XMB, S4, WL, GATHER, ATOMIC>), g, b, 0, s, mp); \
    return hipGetLastError();                                                                    \
  }
  XS_CASE(1, true, true) XS_CASE(1, false, true) XS_CASE(2, true, true) XS_CASE(2, false, true)
  XS_CASE(1, true, false) XS_CASE(1, false, false) XS_CASE(2, true, false) XS_CASE(2, false, false)
#undef XS_CASE
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_ffn_mx_stream(const FfnMxArgs &a, hipStream_t s) {
  if (a.R_cap == 0 || a.T == 0) return hipSuccess;
  hipError_t err = hipSuccess;
  // 32-row M tiles while the rows per expert average at most 16, else 64-row tiles
  const int xmb = (long long)a.R_cap <= 16LL * a.El ? 1 : 2;
  const int xbm = 32 * xmb;
  // worst-case M tiles: sum_e ceil(c_e/xbm) <= (R + El*(xbm-1))/xbm and <= El*ceil(T/xbm)
  const long long mt1 = ((long long)a.R_cap + (long long)a.El * (xbm - 1)) / xbm;
  const long long mt2 = (long long)a.El * ceil_div_i(a.T, xbm);
  const long long max_mt = mt1 < mt2 ? mt1 : mt2;
  uint8_t *hq = (uint8_t *)a.ws;
  uint8_t *hs = hq + ffn_mx_h_bytes(a.R_cap, a.I);
  MxsParams mp{};
  mp.tp.offsets = a.offsets;
  mp.tp.row_token = a.row_token;
  mp.tp.row_w = a.row_w;
  mp.tp.El = a.El;
  mp.tp.H = a.H;
  mp.tp.I = a.I;
  mp.tp.R_cap = a.R_cap;
  mp.tp.wpacked = a.wpacked;
  if (a.phase & 1) {
    MxsParams m = mp;
    m.tp.a = a.a;
    m.a_scales = a.a_s;
    m.tp.w = a.wgu;
    m.w_scales = a.wgu_s;
    m.tp.out = hq;
    m.out_scales = hs;
    const int nt = ceil_div_i(a.I, XCOLS);
    err = a.gather ? launch_xs<0, true, false>(m, xmb, max_mt, nt, s) : launch_xs<0, false, false>(m, xmb, max_mt, nt, s);
    if (err != hipSuccess) return err;
  }
  if (a.phase & 2) {
    MxsParams m = mp;
    m.tp.a = hq;
    m.a_scales = hs;
    m.tp.w = a.wd;
    m.w_scales = a.wd_s;
    const bool atomic = a.y != nullptr;
    m.tp.out = atomic ? (void *)a.y : (void *)a.y_perm;
    const int nt = ceil_div_i(a.H, 2 * XCOLS);  // down: 64 columns per wave
    err = atomic ? launch_xs<1, false, true>(m, xmb, max_mt, nt, s) : launch_xs<1, false, false>(m, xmb, max_mt, nt, s);
  }
  return err;
}

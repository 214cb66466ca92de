// Weight-streaming MFMA core of the small-batch expert kernels (ffn_stream.hip, decode_fused.hip).
//
// One wave owns NB blocks of 32 weight rows and up to SMB blocks of 32 activation rows.  Every
// lane streams its weight rows straight from HBM into registers in the operand layout of
// v_mfma_f32_32x32x16_bf16: the contraction index may be permuted freely as long as both operands
// use the same permutation, so in every 64-wide k chunk lane (n, g) reads 64 contiguous bytes of
// row n at k offset 32g (bf16; 32 bytes for e4m3) and feeds them to four MFMAs; the two lanes of
// a row cover one whole 128-byte line (in the packed bf16 layout the wave reads 1 KB contiguously
// per load instead).  The activations are read with the same layout.  Two
// chunks are in flight per wave (register double buffering).
#pragma once
#include "common.h"

namespace sc {

// 8 bf16 operands from 16 bytes of bf16, or from 8 bytes of e4m3 (exact conversion).
template <bool FP8>
__device__ __forceinline__ bf16x8_t as_operand(const u32x4_t *q, int s) {
  if constexpr (FP8) {
    // q[0] holds k 0..15, q[1] k 16..31 of this lane's 32-element slice
    const u32x4_t v = q[s >> 1];
    const uint32_t w0 = (s & 1) ? v.z : v.x, w1 = (s & 1) ? v.w : v.y;
    uint2 a = e4m3x4_to_bf16x4(w0), b = e4m3x4_to_bf16x4(w1);
    u32x4_t r = {a.x, a.y, b.x, b.y};
    return __builtin_bit_cast(bf16x8_t, r);
  } else {
    return __builtin_bit_cast(bf16x8_t, q[s]);
  }
}

// acc[mb][b] += A_mb . W_b^T over KC consecutive 64-wide k chunks.  wrow[b]: this lane's first
// 16-byte weight piece at the first chunk (row n = lane % 32 of block b, k offset 32 (lane / 32)
// elements); pstep: bytes from one of the lane's pieces of a chunk to the next; cstep: bytes from
// one chunk of a row to the next (row-major or packed layout).  arow[mb]: this
// lane's bf16 activation row of block mb at the first chunk, k offset 32 (lane / 32); chunks are
// 64 elements apart.  two_m (wave-uniform): the second activation block is used.
template <bool FP8, int SMB, int NB>
__device__ __forceinline__ void stream_mfma(const char *const (&wrow)[NB], size_t pstep, size_t cstep,
                                            const uint16_t *const (&arow)[SMB], bool two_m, int KC,
                                            f32x16_t (&acc)[SMB][NB]) {
  constexpr int WQ = FP8 ? 2 : 4;  // 16-byte weight loads per lane per 64-wide k chunk
  u32x4_t wq[2][NB][WQ], aq[2][SMB][4];
  auto load = [&](int buf, int k0) __attribute__((always_inline)) {  // k0: first k of the chunk
#pragma unroll
    for (int b = 0; b < NB; b++)
#pragma unroll
      for (int q = 0; q < WQ; q++) wq[buf][b][q] = *(const u32x4_t *)(wrow[b] + (size_t)(k0 >> 6) * cstep + pstep * q);
#pragma unroll
    for (int q = 0; q < 4; q++) aq[buf][0][q] = *(const u32x4_t *)(arow[0] + k0 + 8 * q);
    if constexpr (SMB > 1) {
      if (two_m) {
#pragma unroll
        for (int q = 0; q < 4; q++) aq[buf][SMB - 1][q] = *(const u32x4_t *)(arow[SMB - 1] + k0 + 8 * q);
      }
    }
  };
  auto compute = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < 4; s++) {
      bf16x8_t bo[NB];
#pragma unroll
      for (int b = 0; b < NB; b++) bo[b] = as_operand<FP8>(wq[buf][b], s);
      const bf16x8_t a0 = __builtin_bit_cast(bf16x8_t, aq[buf][0][s]);
#pragma unroll
      for (int b = 0; b < NB; b++) acc[0][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, bo[b], acc[0][b], 0, 0, 0);
      if constexpr (SMB > 1) {
        if (two_m) {
          const bf16x8_t a1 = __builtin_bit_cast(bf16x8_t, aq[buf][SMB - 1][s]);
#pragma unroll
          for (int b = 0; b < NB; b++)
            acc[SMB - 1][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, bo[b], acc[SMB - 1][b], 0, 0, 0);
        }
      }
    }
  };
  if (KC > 0) load(0, 0);
  int kc = 0;
  for (; kc + 2 <= KC; kc += 2) {
    load(1, (kc + 1) * 64);
    compute(0);
    if (kc + 2 < KC) load(0, (kc + 2) * 64);
    compute(1);
  }
  if (kc < KC) compute(0);
}

template <int SMB, int NB>
__device__ __forceinline__ void zero_acc(f32x16_t (&acc)[SMB][NB]) {
#pragma unroll
  for (int mb = 0; mb < SMB; mb++)
#pragma unroll
    for (int b = 0; b < NB; b++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[mb][b][r] = 0.0f;
}

// Row of the 32-row block that accumulator element r of lane ``lane`` holds (its column is lane % 32).
__device__ __forceinline__ int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

}  // namespace sc

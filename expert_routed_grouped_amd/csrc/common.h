// Shared device helpers and internal launcher declarations of the gfx950 MoE library.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#define MOE_WAVE 64

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// bf16 bit patterns held two per 32-bit word: element 0 in the low half.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16 with round-to-nearest-even (hardware conversion on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(uint16_t, b);
}

// Pack two fp32 into two bf16 (lo = a, hi = b), RNE.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16);
}

// Four e4m3 codes (one 32-bit word) -> four bf16 values (two words), exact.
__device__ __forceinline__ uint2 e4m3x4_to_bf16x4(uint32_t w) {
  auto lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  auto hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
  return make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
}

__device__ __forceinline__ float silu_f32(float g) { return g / (1.0f + expf(-g)); }
// SiLU for the bf16 epilogues, whose result is rounded to bf16 right after: hardware exp2 and
// reciprocal (about 1 ulp of fp32 each) instead of the correctly rounded expf and division.
// Limits hold: g -> -inf gives -0 (exp2 -> inf, rcp -> 0), g -> +inf gives g.
__device__ __forceinline__ float silu_fast(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * g));
}

static inline int ceil_div_i(int a, int b) { return (a + b - 1) / b; }
static inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// ---------------------------------------------------------------------------
// Internal launchers (host side).  Arguments are validated by the ABI layer.
// ---------------------------------------------------------------------------
hipError_t launch_route(const void *x, int x_bf16, const void *w, int w_bf16, const float *bias, int T, int H, int E,
                        int k, int32_t *ids, float *gates, hipStream_t s);

size_t permute_ws_bytes(int T, int k, int El);
hipError_t launch_permute(const int32_t *ids, const float *w, int T, int k, int lo, int El, int32_t *counts,
                          int32_t *offsets, int32_t *row_token, float *row_w, int32_t *token_row, int32_t *ws,
                          hipStream_t s);

hipError_t launch_gather_rows(const void *x, int esz, int H, const int32_t *offsets, int El, const int32_t *row_token,
                              int R_cap, void *x_perm, hipStream_t s);

hipError_t launch_combine(const float *y_perm, const int32_t *token_row, const float *w, int T, int k, int H, float *y,
                          hipStream_t s);

hipError_t launch_zero_f32(float *p, size_t n, hipStream_t s);

// Decode route + local dispatch (+ zeroing of the fused-combine target) in one launch.
// Fits for T <= kRouteDispatchMaxT, T*k <= 8192, E <= 256, H % 8 == 0 (H <= 16384) and
// 16-byte aligned x and router weight.  ``ticket`` is a device counter that must be zero
// before the first launch; every launch leaves it zero.
constexpr int kRouteDispatchMaxT = 512;
bool route_dispatch_fits(int T, int H, int E, int k, const void *x, const void *w);
hipError_t launch_route_dispatch(const void *x, int x_bf16, const void *w, int w_bf16, const float *bias, int T, int H,
                                 int E, int k, int lo, int El, int32_t *ids, float *gates, int32_t *counts,
                                 int32_t *offsets, int32_t *row_token, float *row_w, int32_t *token_row,
                                 float *y_zero, uint32_t *ticket, hipStream_t s);

// Fused decode layer (decode_fused.hip): routing, grouping, gate/up and down + combine in one
// persistent launch.  Its workspace starts with uint32 control words (the work queue, the routing
// ticket, the ``routed`` flag, the exit count, an error word and one completion count per local
// expert), zero before the call and zero again after it (the error word excepted), then h
// [El, T, I] bf16 (every token of every local expert).
enum : int { kDecQueue = 0, kDecTicket = 1, kDecRouted = 2, kDecExit = 3, kDecError = 4, kDecDone = 64 };
constexpr int kDecodeLayerMaxT = 64;  // every token of the batch fits one 64-row tile
struct DecodeArgs {
  const void *x;            // [T, H] bf16
  const void *wr;           // router weight
  int wmode;                // 0 fp32 [E, H], 1 bf16 [E, H], 2 fp32 packed [H/4, E, 4]
  const float *bias;        // [E] or NULL
  int T, H, E, k, lo, El, I;
  int32_t *ids;
  float *gates;
  int32_t *counts, *offsets, *row_token;
  float *row_w;
  int32_t *token_row;
  float *y;                 // [T, H] fp32, overwritten
  const void *wgu, *wd;     // expert weights (bf16 or e4m3)
  const float *sgu, *sd;    // e4m3 per-channel scales
  int fp8, wpacked;
  void *ws;                 // decode_layer_ws_bytes(T, k, El, I) bytes, 256-byte aligned (T <= kDecodeLayerMaxT)
};
size_t decode_layer_ws_bytes(int T, int k, int El, int I);
hipError_t launch_decode_layer(const DecodeArgs &a, hipStream_t s);

// Row maps of one group holding every token once, in order: offsets = {0, T},
// row_token[i] = i, row_w[i] = 1 (the shared expert as a one-expert grouped FFN).
hipError_t launch_identity_rows(int T, int32_t *offsets, int32_t *row_token, float *row_w, hipStream_t s);

// Grouped FFN.  ``h`` is the intermediate [R_cap, I] (bf16 or fp32 by path).
struct FfnArgs {
  const void *a;          // x [T,H] (gather) or x_perm [R_cap,H]
  int a_bf16;             // 1: bf16 activations, 0: fp32
  int gather;             // 1: row r reads a[row_token[r]]
  const int32_t *offsets; // [El+1]
  const int32_t *row_token;
  const float *row_w;
  int El, T, R_cap, H, I;
  const void *w_gu;       // [El, 2I, H]
  const void *w_d;        // [El, H, I]
  int w_dt;               // 0 f32, 1 bf16, 2 e4m3
  const float *s_gu, *s_d;
  float *y;               // fused combine target (atomic) or NULL
  float *y_perm;          // per-row outputs when y == NULL
  void *h;                // intermediate
  int phase;              // bit 0: gate/up half, bit 1: down half
  int kernel;             // bf16 / fp8 weights: 0 pick by rows per expert, 1 weight streaming, 2 tiles
  int wpacked;            // both weight tensors in the packed block layout (moe_pack_weights)
  int ksplit;             // weight streaming only: split K over this many workgroups per tile (needs y and
  float *gu32;            // gu32, an fp32 [R_cap, 2I] scratch for the G and U partial sums)
};

hipError_t launch_ffn(const FfnArgs &a, hipStream_t s);

// Repack row-major weights [E, N, K] (esz-byte elements, N % 32 == 0, K % 64 == 0) into the
// packed block layout read by the FFN kernels when FfnArgs::wpacked is set.
hipError_t launch_pack_weights(const void *w, int esz, int E, int N, int K, void *packed, hipStream_t s);

// MXFP8 quantisation of rows x K values (K % 32 == 0).
hipError_t launch_quantize_mx(const void *x, int x_bf16, int rows, int K, uint8_t *codes, uint8_t *scales,
                              hipStream_t s);

// W8A8 MXFP8 grouped FFN.  ``ws`` holds h as MXFP8: R_cap*I codes (ffn_mx_h_bytes)
// followed by R_cap*I/32 scale bytes.
struct FfnMxArgs {
  const uint8_t *a, *a_s;      // activation codes [rows, H] and scales [rows, H/32]
  int gather;                  // 1: row r reads a[row_token[r]]
  const int32_t *offsets;      // [El+1]
  const int32_t *row_token;
  const float *row_w;
  int El, T, R_cap, H, I;
  const uint8_t *wgu, *wgu_s;  // [El, 2I, H], [El, 2I, H/32]
  const uint8_t *wd, *wd_s;    // [El, H, I], [El, H, I/32]
  float *y, *y_perm;
  void *ws;
  int phase;                   // bit 0: gate/up half, bit 1: down half
  int kernel;                  // 0 pick by rows per expert, 1 weight streaming, 2 tiles
  int wpacked;                 // weight codes in the packed block layout (moe_pack_weights)
};
size_t ffn_mx_h_bytes(int R_cap, int I);
hipError_t launch_ffn_mx(const FfnMxArgs &a, hipStream_t s);
// Weight-streaming W8A8 path for small batches (ffn_mx_stream.hip).
hipError_t launch_ffn_mx_stream(const FfnMxArgs &a, hipStream_t s);

// C ABI of the MoE layer library: argument checks on the host, then launches.
// Every check runs before anything is enqueued, so an error return means the
// stream is untouched.  No call allocates, frees or synchronises.
#include "../../include/moe.h"
#include "common.h"

#include <mutex>

#ifndef SHARED_SPLIT_WG
#define SHARED_SPLIT_WG 192  // measured on the 64-token decode batch (I_s = 1536): 1024 -> 72 us, 384 -> 72, 192 -> 55, 96 -> 57, 48 -> 74
#endif

#define MOE_VERSION_NUMBER 100  // 0.1.0

constexpr int kMaxExperts = 1024;  // experts of a layer (routing) and local experts of a call

// Intermediate h of moe_grouped_ffn_noalloc, for callers that cannot allocate device memory.  Each
// GPU the library runs on holds its own copy until the process ends; host code never passes the
// array's name to a kernel (on the host it is only a stand-in), always the device address that
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

inline bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
inline int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];  // device address of ``scratch`` per device, looked up once

// Device address of the current device's copy of ``scratch``; the first call on a device looks it up
// with that device current and keeps it.
int scratch_for_current_device(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return MOE_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

// defined in route.hip (C++ linkage, outside the C ABI)
hipError_t launch_pack_router(const void *w, int w_bf16, int E, int H, float *out, hipStream_t s);  // route.hip

extern "C" {

int moe_version(void) { return MOE_VERSION_NUMBER; }

const char *moe_status_str(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "a required pointer is NULL";
    case MOE_ERR_SHAPE: return "a size is out of the supported range";
    case MOE_ERR_DTYPE: return "unsupported element type or type combination";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_HIP: return "a kernel launch failed";
    case MOE_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    default: return "unknown status";
  }
}

size_t moe_workspace_size(int op, int T, int k, int E_loc, int H, int I) {
  if (T < 0 || k < 1 || E_loc < 1 || H < 1 || I < 1) return 0;
  const int R_cap = (int)((long long)T * (k < E_loc ? k : E_loc));
  switch (op) {
    case MOE_OP_PERMUTE: return moe_permute_workspace_size(T, k, E_loc);
    case MOE_OP_GROUPED_FFN: return moe_ffn_workspace_size(R_cap, E_loc, H, I, MOE_BF16);
    case MOE_OP_GROUPED_FFN_F32: return moe_ffn_workspace_size(R_cap, E_loc, H, I, MOE_F32);
    case MOE_OP_GROUPED_FFN_MX: return moe_ffn_mx_workspace_size(R_cap, I);
    case MOE_OP_ROUTE_DISPATCH: return moe_route_dispatch_workspace_size();
    case MOE_OP_DECODE_LAYER: return moe_decode_layer_workspace_size(T, k, E_loc, I);
    case MOE_OP_SHARED_EXPERT: return moe_shared_workspace_size(T, I, MOE_BF16);
    case MOE_OP_SHARED_EXPERT_F32: return moe_shared_workspace_size(T, I, MOE_F32);
    default: return 0;
  }
}

int moe_route(const void *x, int x_dtype, const void *w_router, int w_dtype, const float *bias, int T, int H, int E,
              int k, int32_t *topk_ids, float *topk_w, void *stream) {
  if (T < 0 || H < 1 || E < 1 || E > kMaxExperts || k < 1 || k > E || k > 32) return MOE_ERR_SHAPE;
  if ((long long)T * k >= (1LL << 31) || (long long)T * H >= (1LL << 40)) return MOE_ERR_SHAPE;
  if ((x_dtype != MOE_F32 && x_dtype != MOE_BF16) || (w_dtype != MOE_F32 && w_dtype != MOE_BF16)) return MOE_ERR_DTYPE;
  if (T == 0) return MOE_OK;
  if (!x || !w_router || !topk_ids || !topk_w) return MOE_ERR_NULL;
  return hip_status(launch_route(x, x_dtype == MOE_BF16, w_router, w_dtype == MOE_BF16, bias, T, H, E, k, topk_ids,
                                 topk_w, (hipStream_t)stream));
}

size_t moe_route_dispatch_workspace_size(void) { return 256; }

int moe_pack_router(const void *w_router, int w_dtype, int E, int H, float *out, void *stream) {
  if (E < 1 || E > kMaxExperts || H < 4 || H % 4 != 0) return MOE_ERR_SHAPE;
  if (w_dtype != MOE_F32 && w_dtype != MOE_BF16) return MOE_ERR_DTYPE;
  if (!w_router || !out) return MOE_ERR_NULL;
  if (((uintptr_t)w_router & (w_dtype == MOE_BF16 ? 1u : 3u)) != 0 || !aligned16(out)) return MOE_ERR_ALIGN;
  return hip_status(launch_pack_router(w_router, w_dtype == MOE_BF16, E, H, out, (hipStream_t)stream));
}

int moe_route_dispatch(const void *x, int x_dtype, const void *w_router, int w_dtype, const float *bias, int T, int H,
                       int E, int k, int e_begin, int e_end, int32_t *topk_ids, float *topk_w, int32_t *counts,
                       int32_t *offsets, int32_t *row_token, float *row_w, int32_t *token_row, float *y_zero,
                       void *workspace, size_t workspace_bytes, void *stream) {
  if (T < 0 || H < 1 || E < 1 || E > kMaxExperts || k < 1 || k > E || k > 32) return MOE_ERR_SHAPE;
  if (e_begin < 0 || e_end <= e_begin || e_end > E) return MOE_ERR_SHAPE;
  if ((x_dtype != MOE_F32 && x_dtype != MOE_BF16) ||
      (w_dtype != MOE_F32 && w_dtype != MOE_BF16 && w_dtype != MOE_F32_ROUTER_PACKED))
    return MOE_ERR_DTYPE;
  if (!counts || !offsets) return MOE_ERR_NULL;
  if (T > 0 && (!x || !w_router || !topk_ids || !topk_w || !row_token || !row_w || !token_row)) return MOE_ERR_NULL;
  if (T > 0 && !route_dispatch_fits(T, H, E, k, x, w_router)) return MOE_ERR_SHAPE;
  if (y_zero && (H % 4 != 0 || !aligned16(y_zero))) return MOE_ERR_ALIGN;
  if (!workspace || workspace_bytes < moe_route_dispatch_workspace_size()) return MOE_ERR_WORKSPACE;
  if (((uintptr_t)workspace & 255u) != 0) return MOE_ERR_ALIGN;
  if (T == 0)  // nothing to route: zero counts and offsets as moe_permute does
    return hip_status(launch_permute(nullptr, nullptr, 0, k, e_begin, e_end - e_begin, counts, offsets, row_token,
                                     row_w, token_row, nullptr, (hipStream_t)stream));
  const int w_mode = w_dtype == MOE_BF16 ? 1 : (w_dtype == MOE_F32_ROUTER_PACKED ? 2 : 0);
  return hip_status(launch_route_dispatch(x, x_dtype == MOE_BF16, w_router, w_mode, bias, T, H, E, k,
                                          e_begin, e_end - e_begin, topk_ids, topk_w, counts, offsets, row_token,
                                          row_w, token_row, y_zero, (uint32_t *)workspace, (hipStream_t)stream));
}

size_t moe_decode_layer_workspace_size(int T, int k, int E_loc, int I) {
  if (T < 0 || k < 1 || E_loc < 1 || I < 1) return 0;
  return decode_layer_ws_bytes(T, k, E_loc, I);
}

int moe_decode_layer(const void *x, int x_dtype, const void *w_router, int wr_dtype, const float *bias, int T, int H,
                     int E, int k, int e_begin, int e_end, int I, const void *w_gate_up, const void *w_down,
                     int w_dtype, const float *s_gate_up, const float *s_down, int32_t *topk_ids, float *topk_w,
                     int32_t *counts, int32_t *offsets, int32_t *row_token, float *row_w, int32_t *token_row,
                     float *y, void *workspace, size_t workspace_bytes, unsigned flags, void *stream) {
  if (T < 0 || H < 64 || I < 64 || H % 64 != 0 || I % 64 != 0 || E < 1 || E > 256 || k < 1 || k > E || k > 32)
    return MOE_ERR_SHAPE;
  if (e_begin < 0 || e_end <= e_begin || e_end > E) return MOE_ERR_SHAPE;
  if (T > kDecodeLayerMaxT || H > 16384 || (long long)H * I >= (1LL << 30)) return MOE_ERR_SHAPE;
  if (x_dtype != MOE_BF16) return MOE_ERR_DTYPE;
  if (wr_dtype != MOE_F32 && wr_dtype != MOE_BF16 && wr_dtype != MOE_F32_ROUTER_PACKED) return MOE_ERR_DTYPE;
  if (w_dtype != MOE_BF16 && w_dtype != MOE_FP8_E4M3) return MOE_ERR_DTYPE;
  if ((flags & ~MOE_FFN_PACKED_WEIGHTS) != 0) return MOE_ERR_SHAPE;
  if (!counts || !offsets) return MOE_ERR_NULL;
  if (T > 0 && (!x || !w_router || !w_gate_up || !w_down || !topk_ids || !topk_w || !row_token || !row_w ||
                !token_row || !y))
    return MOE_ERR_NULL;
  if (T > 0 && w_dtype == MOE_FP8_E4M3 && (!s_gate_up || !s_down)) return MOE_ERR_NULL;
  const int El = e_end - e_begin;
  if (!workspace || workspace_bytes < decode_layer_ws_bytes(T, k, El, I)) return MOE_ERR_WORKSPACE;
  if (((uintptr_t)workspace & 255u) != 0) return MOE_ERR_ALIGN;
  if (T == 0)  // nothing to route: zero counts and offsets as moe_permute does
    return hip_status(launch_permute(nullptr, nullptr, 0, k, e_begin, El, counts, offsets, row_token, row_w,
                                     token_row, nullptr, (hipStream_t)stream));
  if (!aligned16(x) || !aligned16(w_router) || !aligned16(w_gate_up) || !aligned16(w_down) || !aligned16(y))
    return MOE_ERR_ALIGN;
  DecodeArgs a{};
  a.x = x;
  a.wr = w_router;
  a.wmode = wr_dtype == MOE_BF16 ? 1 : (wr_dtype == MOE_F32_ROUTER_PACKED ? 2 : 0);
  a.bias = bias;
  a.T = T;
  a.H = H;
  a.E = E;
  a.k = k;
  a.lo = e_begin;
  a.El = El;
  a.I = I;
  a.ids = topk_ids;
  a.gates = topk_w;
  a.counts = counts;
  a.offsets = offsets;
  a.row_token = row_token;
  a.row_w = row_w;
  a.token_row = token_row;
  a.y = y;
  a.wgu = w_gate_up;
  a.wd = w_down;
  a.sgu = s_gate_up;
  a.sd = s_down;
  a.fp8 = w_dtype == MOE_FP8_E4M3;
  a.wpacked = (flags & MOE_FFN_PACKED_WEIGHTS) != 0;
  a.ws = workspace;
  return hip_status(launch_decode_layer(a, (hipStream_t)stream));
}

int moe_permute(const int32_t *topk_ids, const float *topk_w, int T, int k, int E, int e_begin, int e_end,
                int32_t *counts, int32_t *offsets, int32_t *row_token, float *row_w, int32_t *token_row,
                const void *x, int x_dtype, int H, void *x_perm, void *workspace, size_t workspace_bytes,
                void *stream) {
  if (T < 0 || E < 1 || E > kMaxExperts || k < 1 || k > E || k > 32) return MOE_ERR_SHAPE;
  if (e_begin < 0 || e_end <= e_begin || e_end > E) return MOE_ERR_SHAPE;
  if ((long long)T * k >= (1LL << 31)) return MOE_ERR_SHAPE;
  if (!counts || !offsets) return MOE_ERR_NULL;
  if (T > 0 && (!topk_ids || !topk_w || !row_token || !row_w || !token_row)) return MOE_ERR_NULL;
  const bool gather = x != nullptr || x_perm != nullptr;
  if (gather) {
    if (!x || !x_perm) return MOE_ERR_NULL;
    if (x_dtype != MOE_F32 && x_dtype != MOE_BF16) return MOE_ERR_DTYPE;
    if (H < 8 || H % 8 != 0) return MOE_ERR_SHAPE;
    if (!aligned16(x) || !aligned16(x_perm)) return MOE_ERR_ALIGN;
  }
  const int El = e_end - e_begin;
  if (!workspace || workspace_bytes < permute_ws_bytes(T, k, El)) return MOE_ERR_WORKSPACE;
  if (((uintptr_t)workspace & 255u) != 0) return MOE_ERR_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  hipError_t err = launch_permute(topk_ids, topk_w, T, k, e_begin, El, counts, offsets, row_token, row_w, token_row,
                                  (int32_t *)workspace, s);
  if (err != hipSuccess) return MOE_ERR_HIP;
  if (gather && T > 0) {
    const int R_cap = T * (k < El ? k : El);
    err = launch_gather_rows(x, x_dtype == MOE_BF16 ? 2 : 4, H, offsets, El, row_token, R_cap, x_perm, s);
  }
  return hip_status(err);
}

size_t moe_permute_workspace_size(int T, int k, int E_loc) {
  if (T < 0 || k < 1 || E_loc < 1) return 0;
  return permute_ws_bytes(T, k, E_loc);
}

size_t moe_ffn_workspace_size(int R_cap, int E_loc, int H, int I, int a_dtype) {
  (void)H;
  if (R_cap < 0 || E_loc < 1 || I < 1) return 0;
  const size_t esz = a_dtype == MOE_F32 ? 4 : 2;
  return align_up((size_t)R_cap * (size_t)I * esz, 256);
}

}  // extern "C"

namespace {

// Checks and launches of moe_grouped_ffn, whose intermediate h lives in ``workspace`` or, with
// ``static_scratch``, in the current device's copy of ``scratch`` (looked up after every check passed).
int grouped_ffn(const void *a, int a_dtype, const int32_t *offsets, const int32_t *row_token, const float *row_w,
                int E_loc, int T, int R_cap, int H, int I, const void *w_gate_up, const void *w_down, int w_dtype,
                const float *s_gate_up, const float *s_down, float *y, float *y_perm, void *workspace,
                size_t workspace_bytes, unsigned flags, void *stream, bool static_scratch = false) {
  if (static_scratch) workspace_bytes = MOE_NOALLOC_SCRATCH_BYTES;
  if (T < 0 || R_cap < 0 || E_loc < 1 || E_loc > kMaxExperts || H < 64 || I < 64 || H % 64 != 0 || I % 64 != 0)
    return MOE_ERR_SHAPE;
  if ((long long)R_cap > (long long)T * E_loc) return MOE_ERR_SHAPE;
  // the tile kernels address a row-major operand with 32-bit byte offsets (rows x dim x 4 < 2^32)
  if ((long long)(T > R_cap ? T : R_cap) * (H > I ? H : I) >= (1LL << 30) || (long long)H * I >= (1LL << 30))
    return MOE_ERR_SHAPE;
  const bool bf16_path = a_dtype == MOE_BF16 && (w_dtype == MOE_BF16 || w_dtype == MOE_FP8_E4M3);
  const bool f32_path = a_dtype == MOE_F32 && w_dtype == MOE_F32;
  if (!bf16_path && !f32_path) return MOE_ERR_DTYPE;
  if ((y == nullptr) == (y_perm == nullptr)) return MOE_ERR_NULL;
  const bool gather = (flags & MOE_FFN_GATHER) != 0;
  if (!a || !offsets || !w_gate_up || !w_down) return MOE_ERR_NULL;
  if ((gather || y) && !row_token) return MOE_ERR_NULL;
  if (y && !row_w) return MOE_ERR_NULL;
  if (w_dtype == MOE_FP8_E4M3 && (!s_gate_up || !s_down)) return MOE_ERR_NULL;
  if (!workspace && !static_scratch) return MOE_ERR_WORKSPACE;
  if (workspace_bytes < moe_ffn_workspace_size(R_cap, E_loc, H, I, a_dtype)) return MOE_ERR_WORKSPACE;
  if (!aligned16(a) || !aligned16(w_gate_up) || !aligned16(w_down) || (y && !aligned16(y)) ||
      (y_perm && !aligned16(y_perm)) || ((uintptr_t)workspace & 255u) != 0)
    return MOE_ERR_ALIGN;
  const unsigned only = flags & (MOE_FFN_ONLY_GATE_UP | MOE_FFN_ONLY_DOWN);
  if (only == (MOE_FFN_ONLY_GATE_UP | MOE_FFN_ONLY_DOWN)) return MOE_ERR_SHAPE;
  if ((flags & ~(MOE_FFN_GATHER | MOE_FFN_ZERO_Y | MOE_FFN_ONLY_GATE_UP | MOE_FFN_ONLY_DOWN |
                 MOE_FFN_PACKED_WEIGHTS)) != 0)
    return MOE_ERR_SHAPE;
  const bool packed = (flags & MOE_FFN_PACKED_WEIGHTS) != 0;
  if (packed && w_dtype == MOE_F32) return MOE_ERR_DTYPE;
  if (static_scratch) {
    const int st = scratch_for_current_device(&workspace);
    if (st != MOE_OK) return st;
  }
  hipStream_t s = (hipStream_t)stream;
  if (y && (flags & MOE_FFN_ZERO_Y) && only != MOE_FFN_ONLY_GATE_UP) {
    hipError_t err = launch_zero_f32(y, (size_t)T * H, s);
    if (err != hipSuccess) return MOE_ERR_HIP;
  }
  FfnArgs fa{};
  fa.a = a;
  fa.a_bf16 = a_dtype == MOE_BF16;
  fa.gather = gather;
  fa.offsets = offsets;
  fa.row_token = row_token;
  fa.row_w = row_w;
  fa.El = E_loc;
  fa.T = T;
  fa.R_cap = R_cap;
  fa.H = H;
  fa.I = I;
  fa.w_gu = w_gate_up;
  fa.w_d = w_down;
  fa.w_dt = w_dtype == MOE_F32 ? 0 : (w_dtype == MOE_BF16 ? 1 : 2);
  fa.s_gu = s_gate_up;
  fa.s_d = s_down;
  fa.y = y;
  fa.y_perm = y_perm;
  fa.h = workspace;
  fa.phase = only == MOE_FFN_ONLY_GATE_UP ? 1 : (only == MOE_FFN_ONLY_DOWN ? 2 : 3);
  fa.wpacked = packed;
  return hip_status(launch_ffn(fa, s));
}

}  // namespace

extern "C" {

int moe_grouped_ffn(const void *a, int a_dtype, const int32_t *offsets, const int32_t *row_token, const float *row_w,
                    int E_loc, int T, int R_cap, int H, int I, const void *w_gate_up, const void *w_down, int w_dtype,
                    const float *s_gate_up, const float *s_down, float *y, float *y_perm, void *workspace,
                    size_t workspace_bytes, unsigned flags, void *stream) {
  return grouped_ffn(a, a_dtype, offsets, row_token, row_w, E_loc, T, R_cap, H, I, w_gate_up, w_down, w_dtype,
                     s_gate_up, s_down, y, y_perm, workspace, workspace_bytes, flags, stream);
}

int moe_grouped_ffn_noalloc(const void *a, int a_dtype, const int32_t *offsets, const int32_t *row_token,
                            const float *row_w, int E_loc, int T, int R_cap, int H, int I, const void *w_gate_up,
                            const void *w_down, int w_dtype, const float *s_gate_up, const float *s_down, float *y,
                            float *y_perm, unsigned flags, void *stream) {
  // the intermediate h goes to this GPU's copy of the static scratch array; sizes whose h does not
  // fit it are refused (MOE_ERR_WORKSPACE) with the other argument errors, before anything is enqueued
  return grouped_ffn(a, a_dtype, offsets, row_token, row_w, E_loc, T, R_cap, H, I, w_gate_up, w_down, w_dtype,
                     s_gate_up, s_down, y, y_perm, nullptr, 0, flags, stream, true);
}

int moe_pack_weights(const void *w, int w_dtype, int E, int N, int K, void *packed, void *stream) {
  if (w_dtype != MOE_BF16 && w_dtype != MOE_FP8_E4M3) return MOE_ERR_DTYPE;
  if (E < 1 || N < 32 || K < 64 || N % 32 != 0 || K % 64 != 0) return MOE_ERR_SHAPE;
  if (!w || !packed) return MOE_ERR_NULL;
  if (!aligned16(w) || !aligned16(packed)) return MOE_ERR_ALIGN;
  const int esz = w_dtype == MOE_BF16 ? 2 : 1;
  const size_t bytes = (size_t)E * (size_t)N * (size_t)K * (size_t)esz;
  const uintptr_t a0 = (uintptr_t)w, b0 = (uintptr_t)packed;
  if (a0 < b0 + bytes && b0 < a0 + bytes) return MOE_ERR_SHAPE;  // the two buffers overlap
  return hip_status(launch_pack_weights(w, esz, E, N, K, packed, (hipStream_t)stream));
}

// Up to this many tokens the shared expert streams its weights (every token in one or two 64-row
// tiles) with K split over enough workgroups to keep HBM busy; above it the tile kernels run.
constexpr int SHARED_STREAM_ROWS = 128;

size_t moe_shared_workspace_size(int T, int I_s, int a_dtype) {
  if (T < 0 || I_s < 1) return 0;
  const size_t esz = a_dtype == MOE_F32 ? 4 : 2;
  // h [T, I_s], the identity row maps (offsets {0, T}, row_token [T], row_w [T]), then for a
  // decode-sized batch the fp32 G/U partial sums of the split-K gate/up projection [T, 2 I_s]
  size_t b = align_up((size_t)T * (size_t)I_s * esz, 256) + 256 + 2 * align_up((size_t)T * 4, 256);
  if (T <= SHARED_STREAM_ROWS) b += align_up((size_t)T * 2 * (size_t)I_s * 4, 256);
  return b;
}

int moe_shared_expert(const void *x, int x_dtype, int T, int H, int I_s, const void *w_gate_up, const void *w_down,
                      int w_dtype, const float *s_gate_up, const float *s_down, float *y, void *workspace,
                      size_t workspace_bytes, unsigned flags, void *stream) {
  if (T < 0 || H < 64 || I_s < 64 || H % 64 != 0 || I_s % 64 != 0) return MOE_ERR_SHAPE;
  if ((long long)T * (H > I_s ? H : I_s) >= (1LL << 30) || (long long)H * I_s >= (1LL << 30)) return MOE_ERR_SHAPE;
  const bool bf16_path = x_dtype == MOE_BF16 && (w_dtype == MOE_BF16 || w_dtype == MOE_FP8_E4M3);
  const bool f32_path = x_dtype == MOE_F32 && w_dtype == MOE_F32;
  if (!bf16_path && !f32_path) return MOE_ERR_DTYPE;
  if ((flags & ~(MOE_FFN_ZERO_Y | MOE_FFN_PACKED_WEIGHTS)) != 0) return MOE_ERR_SHAPE;
  if ((flags & MOE_FFN_PACKED_WEIGHTS) && w_dtype == MOE_F32) return MOE_ERR_DTYPE;
  if (T == 0) return MOE_OK;
  if (!x || !w_gate_up || !w_down || !y) return MOE_ERR_NULL;
  if (w_dtype == MOE_FP8_E4M3 && (!s_gate_up || !s_down)) return MOE_ERR_NULL;
  if (!workspace) return MOE_ERR_WORKSPACE;
  if (workspace_bytes < moe_shared_workspace_size(T, I_s, x_dtype)) return MOE_ERR_WORKSPACE;
  if (!aligned16(x) || !aligned16(w_gate_up) || !aligned16(w_down) || !aligned16(y) ||
      ((uintptr_t)workspace & 255u) != 0)
    return MOE_ERR_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  const size_t esz = x_dtype == MOE_F32 ? 4 : 2;
  char *ws = (char *)workspace;
  char *maps = ws + align_up((size_t)T * (size_t)I_s * esz, 256);
  int32_t *offsets = (int32_t *)maps;
  int32_t *row_token = (int32_t *)(maps + 256);
  float *row_w = (float *)(maps + 256 + align_up((size_t)T * 4, 256));
  hipError_t err = launch_identity_rows(T, offsets, row_token, row_w, s);
  if (err == hipSuccess && (flags & MOE_FFN_ZERO_Y)) err = launch_zero_f32(y, (size_t)T * H, s);
  if (err != hipSuccess) return MOE_ERR_HIP;
  FfnArgs fa{};
  fa.a = x;
  fa.a_bf16 = x_dtype == MOE_BF16;
  fa.gather = 0;
  fa.offsets = offsets;
  fa.row_token = row_token;
  fa.row_w = row_w;
  fa.El = 1;
  fa.T = T;
  fa.R_cap = T;
  fa.H = H;
  fa.I = I_s;
  fa.w_gu = w_gate_up;
  fa.w_d = w_down;
  fa.w_dt = w_dtype == MOE_F32 ? 0 : (w_dtype == MOE_BF16 ? 1 : 2);
  fa.s_gu = s_gate_up;
  fa.s_d = s_down;
  fa.y = y;  // every row once with weight 1: the "atomic" add is the single add y + o
  fa.h = workspace;
  fa.phase = 3;
  fa.kernel = T <= SHARED_STREAM_ROWS ? 1 : 2;
  fa.wpacked = (flags & MOE_FFN_PACKED_WEIGHTS) != 0;
  if (T <= SHARED_STREAM_ROWS && x_dtype == MOE_BF16) {
    // one expert gives only I_s / 128 gate/up workgroups per 64-row tile: split K over up to half
    // the 64-wide chunks so that about SHARED_SPLIT_WG workgroups stream the weights
    const int tiles = (T + 63) / 64 * ((I_s + 127) / 128);
    int ks = (SHARED_SPLIT_WG + tiles - 1) / tiles;
    if (ks > H / 128) ks = H / 128;
    fa.ksplit = ks > 1 ? ks : 1;
    fa.gu32 = (float *)(maps + 256 + 2 * align_up((size_t)T * 4, 256));
  }
  return hip_status(launch_ffn(fa, s));
}

int moe_combine(const float *y_perm, const int32_t *token_row, const float *topk_w, int T, int k, int H, float *y,
                void *stream) {
  if (T < 0 || k < 1 || k > 32 || H < 4 || H % 4 != 0) return MOE_ERR_SHAPE;
  if ((long long)T * k >= (1LL << 31)) return MOE_ERR_SHAPE;
  if (T == 0) return MOE_OK;
  if (!y_perm || !token_row || !topk_w || !y) return MOE_ERR_NULL;
  if (!aligned16(y_perm) || !aligned16(y)) return MOE_ERR_ALIGN;
  return hip_status(launch_combine(y_perm, token_row, topk_w, T, k, H, y, (hipStream_t)stream));
}

}  // extern "C"

int moe_quantize_mx(const void *x, int x_dtype, int rows, int K, uint8_t *codes, uint8_t *scales, void *stream) {
  if (rows < 0 || K < 32 || K % 32 != 0 || (long long)rows * K >= (1LL << 40)) return MOE_ERR_SHAPE;
  if (x_dtype != MOE_F32 && x_dtype != MOE_BF16) return MOE_ERR_DTYPE;
  if (rows == 0) return MOE_OK;
  if (!x || !codes || !scales) return MOE_ERR_NULL;
  if (!aligned16(x) || ((uintptr_t)codes & 7u) != 0) return MOE_ERR_ALIGN;  // 16-byte loads, 8-byte stores
  return hip_status(launch_quantize_mx(x, x_dtype == MOE_BF16, rows, K, codes, scales, (hipStream_t)stream));
}

size_t moe_ffn_mx_workspace_size(int R_cap, int I) {
  if (R_cap < 0 || I < 1) return 0;
  return ffn_mx_h_bytes(R_cap, I) + align_up((size_t)R_cap * (size_t)(I / 32), 256);
}

int moe_grouped_ffn_mx(const uint8_t *a_codes, const uint8_t *a_scales, const int32_t *offsets,
                       const int32_t *row_token, const float *row_w, int E_loc, int T, int R_cap, int H, int I,
                       const uint8_t *wgu_codes, const uint8_t *wgu_scales, const uint8_t *wd_codes,
                       const uint8_t *wd_scales, float *y, float *y_perm, void *workspace, size_t workspace_bytes,
                       unsigned flags, void *stream) {
  if (T < 0 || R_cap < 0 || E_loc < 1 || E_loc > kMaxExperts || H < 128 || I < 128 || H % 128 != 0 || I % 128 != 0)
    return MOE_ERR_SHAPE;
  if ((long long)R_cap > (long long)T * E_loc) return MOE_ERR_SHAPE;
  if ((long long)(T > R_cap ? T : R_cap) * (H > I ? H : I) >= (1LL << 30) || (long long)H * I >= (1LL << 30))
    return MOE_ERR_SHAPE;
  if ((y == nullptr) == (y_perm == nullptr)) return MOE_ERR_NULL;
  const bool gather = (flags & MOE_FFN_GATHER) != 0;
  if (!a_codes || !a_scales || !offsets || !wgu_codes || !wgu_scales || !wd_codes || !wd_scales) return MOE_ERR_NULL;
  if ((gather || y) && !row_token) return MOE_ERR_NULL;
  if (y && !row_w) return MOE_ERR_NULL;
  if (!workspace) return MOE_ERR_WORKSPACE;
  if (workspace_bytes < moe_ffn_mx_workspace_size(R_cap, I)) return MOE_ERR_WORKSPACE;
  if (!aligned16(a_codes) || !aligned16(wgu_codes) || !aligned16(wd_codes) || (y && !aligned16(y)) ||
      (y_perm && !aligned16(y_perm)) || ((uintptr_t)workspace & 255u) != 0 || ((uintptr_t)a_scales & 3u) != 0 ||
      ((uintptr_t)wgu_scales & 3u) != 0 || ((uintptr_t)wd_scales & 3u) != 0)
    return MOE_ERR_ALIGN;
  const unsigned only = flags & (MOE_FFN_ONLY_GATE_UP | MOE_FFN_ONLY_DOWN);
  if (only == (MOE_FFN_ONLY_GATE_UP | MOE_FFN_ONLY_DOWN)) return MOE_ERR_SHAPE;
  hipStream_t s = (hipStream_t)stream;
  if (y && (flags & MOE_FFN_ZERO_Y) && only != MOE_FFN_ONLY_GATE_UP) {
    if (launch_zero_f32(y, (size_t)T * H, s) != hipSuccess) return MOE_ERR_HIP;
  }
  FfnMxArgs fa{};
  fa.wpacked = (flags & MOE_FFN_PACKED_WEIGHTS) ? 1 : 0;
  fa.a = a_codes;
  fa.a_s = a_scales;
  fa.gather = gather;
  fa.offsets = offsets;
  fa.row_token = row_token;
  fa.row_w = row_w;
  fa.El = E_loc;
  fa.T = T;
  fa.R_cap = R_cap;
  fa.H = H;
  fa.I = I;
  fa.wgu = wgu_codes;
  fa.wgu_s = wgu_scales;
  fa.wd = wd_codes;
  fa.wd_s = wd_scales;
  fa.y = y;
  fa.y_perm = y_perm;
  fa.ws = workspace;
  fa.phase = only == MOE_FFN_ONLY_GATE_UP ? 1 : (only == MOE_FFN_ONLY_DOWN ? 2 : 3);
  return hip_status(launch_ffn_mx(fa, s));
}

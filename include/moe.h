/*
 * moe.h - C ABI of the MI355X (gfx950) Mixture-of-Experts FFN layer library.
 *
 * One MoE FFN layer, as one GPU's share of the work, is four calls:
 *
 *   moe_route        router GEMM, top-k of E experts, renormalised gates
 *   moe_permute      per-expert counts and offsets, rows grouped by expert
 *   moe_grouped_ffn  SwiGLU expert FFN as grouped GEMMs over the expert rows,
 *                    with the gate-weighted combine fused into the
 *                    down-projection epilogue (or per-row outputs for moe_combine)
 *   moe_combine      gate-weighted gather-sum of per-row outputs to token order
 *
 * plus moe_route_dispatch (the first two calls of a decode batch in one
 * launch), moe_decode_layer (all four of a decode batch in one launch), moe_shared_expert (an always-active expert added to y), the W8A8
 * MXFP8 variant of the expert FFN (moe_quantize_mx, moe_grouped_ffn_mx) and
 * moe_pack_weights / moe_pack_router (one-time reorderings of resident expert
 * and router weights for faster reads), and moe_grouped_ffn_noalloc (the expert
 * FFN for callers that cannot allocate a workspace).
 *
 * The method follows three pages: "AI-infra book, ch. 9 Distributed inference"
 * (section 9.3.4, Fig. 9-16: route, group rows by expert, expert GEMMs, weighted
 * combine; section 9.3.2: the expert is three 4096 x 1536 matrices), "Hosting
 * Qwen on Blackwell" (section "MoE Dispatch - Combine": dispatch groups each
 * expert's tokens into GEMM input buffers and combine is a weighted
 * accumulation; section "Expert parallelism": with replicated inputs a rank only
 * selects the tokens of its local experts) and "PagedAttention, speculative
 * decoding, MoE and Blackwell" (MoE list: a gating network sends each token to
 * its top-K experts).  The library never drops an assignment of a local expert
 * and never changes k (book, section 9.4.2: changing top-k changes the model).
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Every array argument is a DEVICE pointer to row-major memory owned by the
 *    caller.  The library allocates nothing, frees nothing and keeps no mutable
 *    global state (one exception: moe_grouped_ffn_noalloc keeps its intermediate
 *    in a static per-GPU scratch array); calls on different streams may run
 *    concurrently as long as they do not share output buffers.
 *  - ``stream`` is a hipStream_t passed as ``void*`` (NULL = the null stream).
 *    All work is enqueued on it; the calls return without waiting for the GPU.
 *    There is no device-to-host copy anywhere inside the calls.
 *  - Return value: MOE_OK (0) or a negative MOE_ERR_* code.  Argument errors are
 *    detected on the host before anything is enqueued (then nothing ran).
 *    MOE_ERR_HIP means a launch failed (hipGetLastError after the launch).
 *    Faults inside kernels surface, as usual for HIP, at the next
 *    synchronisation of the stream.  NaN/Inf input values are not checked.
 *  - Element types: MOE_F32 (float), MOE_BF16 (bfloat16 bit patterns, uint16),
 *    MOE_FP8_E4M3 (OCP E4M3 codes, uint8; only for expert weights, always with
 *    fp32 per-output-channel scales), MOE_MXFP8 (OCP microscaling: E4M3 codes,
 *    uint8, plus one E8M0 scale byte 2^(s-127) per 32 consecutive values along
 *    the contraction axis, in a separate uint8 array [rows, K/32]; used by
 *    moe_quantize_mx and moe_grouped_ffn_mx).
 *  - Sizes: T >= 0 tokens, hidden H, E experts with 1 <= k <= min(E, 32),
 *    E <= 1024, intermediate I.  Local experts are [e_begin, e_end) with
 *    E_loc = e_end - e_begin >= 1; R_cap = T * min(k, E_loc) bounds the number
 *    of local assignments, so every row buffer is sized without knowing the
 *    routing on the host.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element types */
#define MOE_F32 0
#define MOE_BF16 1
#define MOE_FP8_E4M3 2
#define MOE_MXFP8 3
#define MOE_F32_ROUTER_PACKED 4 /* router weight as written by moe_pack_router (moe_route_dispatch only) */

/* status codes */
#define MOE_OK 0
#define MOE_ERR_NULL (-1)      /* a required pointer is NULL */
#define MOE_ERR_SHAPE (-2)     /* a size is out of the supported range */
#define MOE_ERR_DTYPE (-3)     /* unsupported element type or type combination */
#define MOE_ERR_WORKSPACE (-4) /* workspace missing or too small */
#define MOE_ERR_HIP (-5)       /* a kernel launch failed */
#define MOE_ERR_ALIGN (-6)     /* a pointer is not 16-byte aligned */

/* moe_grouped_ffn flags */
#define MOE_FFN_GATHER 1u /* ``a`` is x [T,H]; row r reads x[row_token[r]] (no x_perm needed) */
#define MOE_FFN_ZERO_Y 2u /* zero y [T,H] on the stream before the fused combine accumulates */
#define MOE_FFN_ONLY_GATE_UP 4u /* run only the first half: gate/up + SwiGLU into the workspace's h */
#define MOE_FFN_ONLY_DOWN 8u    /* run only the second half: down + combine from the workspace's h, which a
                                   preceding MOE_FFN_ONLY_GATE_UP call with the same arguments filled */
#define MOE_FFN_PACKED_WEIGHTS 16u /* w_gate_up and w_down are in the packed block layout that
                                      moe_pack_weights writes (bf16 and fp8 weights only) */

/* moe_workspace_size operations */
#define MOE_OP_PERMUTE 0          /* moe_permute */
#define MOE_OP_GROUPED_FFN 1      /* moe_grouped_ffn / moe_shared_expert with bf16 activations */
#define MOE_OP_GROUPED_FFN_F32 2  /* moe_grouped_ffn / moe_shared_expert with fp32 activations */
#define MOE_OP_GROUPED_FFN_MX 3   /* moe_grouped_ffn_mx */
#define MOE_OP_ROUTE_DISPATCH 4   /* moe_route_dispatch */
#define MOE_OP_DECODE_LAYER 5     /* moe_decode_layer */
#define MOE_OP_SHARED_EXPERT 6    /* moe_shared_expert with bf16 activations (I = I_s, E_loc and k unused) */
#define MOE_OP_SHARED_EXPERT_F32 7 /* moe_shared_expert with fp32 activations */

/* Library version (major*10000 + minor*100 + patch). */
int moe_version(void);

/* Human-readable text of a status code (static storage, never NULL). */
const char *moe_status_str(int status);

/*
 * Bytes of workspace one call of operation ``op`` (MOE_OP_*) needs for T tokens, top-k, E_loc local
 * experts, hidden H and intermediate I (row buffers sized by R_cap = T * min(k, E_loc)); the same
 * numbers as the per-call functions below (moe_permute_workspace_size, moe_ffn_workspace_size,
 * moe_ffn_mx_workspace_size, moe_route_dispatch_workspace_size, moe_decode_layer_workspace_size,
 * moe_shared_workspace_size).  0 for an unknown op or sizes out of range.
 */
size_t moe_workspace_size(int op, int T, int k, int E_loc, int H, int I);

/*
 * moe_route - router GEMM, top-k selection and renormalised gates.
 *
 * Defined by: PagedAttention/MoE page, MoE list (a gating network picks the
 * top-K experts of each token); AI-infra book section 9.3.4 (the router picks 8
 * experts per token, the combine is the routing-weighted sum).
 *
 *   logit[t,e] = fp32 fused-multiply-add chain over h = 0..H-1 (ascending,
 *                starting at +0) of x[t,h] * w_router[e,h], then + bias[e]
 *                (one fp32 add) when bias != NULL.  This order is part of the
 *                contract: it makes the selected experts reproducible bit for bit.
 *   topk_ids[t,0..k-1] = the k experts with the largest logits, largest first;
 *                equal logits (IEEE equality, -0 == +0) go to the lower index.
 *   topk_w[t,j] = exp(l_j - l_0) / sum_i exp(l_i - l_0) over the k selected
 *                logits (= softmax over all E renormalised over the k selected).
 *
 * x [T,H] and w_router [E,H]: MOE_F32 or MOE_BF16 each; bias [E] fp32 or NULL.
 * Outputs topk_ids [T,k] int32 and topk_w [T,k] fp32 are overwritten.
 * Errors: MOE_ERR_NULL (x, w_router, topk_ids or topk_w NULL with T > 0),
 * MOE_ERR_SHAPE (T < 0, H < 1, E < 1 or E > 1024, k < 1, k > min(E, 32)),
 * MOE_ERR_DTYPE, MOE_ERR_HIP.  T == 0 enqueues nothing.
 */
int moe_route(const void *x, int x_dtype, const void *w_router, int w_dtype, const float *bias,
              int T, int H, int E, int k, int32_t *topk_ids, float *topk_w, void *stream);

/*
 * moe_permute - local dispatch: group the assignments of local experts by expert.
 *
 * Defined by: "Hosting Qwen on Blackwell", section "MoE Dispatch - Combine"
 * (dispatch moves and groups tokens for the MoE GEMM) and section "Expert
 * parallelism" (inputs replicated on all ranks, so dispatch only selects the
 * tokens routed to local experts and prepares the GEMM input buffers);
 * AI-infra book section 9.3.4 (rows are permuted by expert before the expert
 * GEMMs); book section 9.4.2 (m_j, the rows each expert receives).
 *
 *   counts[i]  = number of assignments (t, j) with topk_ids[t,j] == e_begin + i
 *   offsets    = exclusive prefix sum of counts, offsets[E_loc] = R
 *   rows r in [offsets[i], offsets[i+1]) are the assignments of expert
 *   e_begin + i in increasing token order (the unique stable order), and
 *   row_token[r] = t, row_w[r] = topk_w[t,j], token_row[t,j] = r;
 *   token_row[t,j] = -1 when topk_ids[t,j] is not local.
 *   x_perm[r,:] = x[row_token[r],:] bit for bit when x and x_perm are not NULL.
 *
 * Sizes: counts [E_loc], offsets [E_loc+1] int32; row_token [R_cap] int32,
 * row_w [R_cap] fp32 (only the first R entries are written); token_row [T,k]
 * int32; x [T,H] and x_perm [R_cap,H] of element type x_dtype (MOE_F32 or
 * MOE_BF16), 16-byte aligned, H a multiple of 8.  topk_ids must hold distinct
 * experts per token in [0, E) (as moe_route writes them).  workspace: at least
 * moe_permute_workspace_size(T, k, E_loc) bytes, 256-byte aligned.
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE (0 <= e_begin < e_end <= E, E <= 1024,
 * 1 <= k <= min(E,32), T*k < 2^31), MOE_ERR_DTYPE, MOE_ERR_ALIGN,
 * MOE_ERR_WORKSPACE, MOE_ERR_HIP.
 */
int moe_permute(const int32_t *topk_ids, const float *topk_w, int T, int k, int E, int e_begin, int e_end,
                int32_t *counts, int32_t *offsets, int32_t *row_token, float *row_w, int32_t *token_row,
                const void *x, int x_dtype, int H, void *x_perm, void *workspace, size_t workspace_bytes,
                void *stream);

/* Bytes of workspace moe_permute needs (per-chunk expert counts of large batches). */
size_t moe_permute_workspace_size(int T, int k, int E_loc);

/*
 * Bytes of workspace moe_grouped_ffn needs (the intermediate h [R_cap, I]), for
 * activations of type a_dtype.
 */
size_t moe_ffn_workspace_size(int R_cap, int E_loc, int H, int I, int a_dtype);

/*
 * moe_grouped_ffn - SwiGLU expert FFN over the grouped rows, with the combine.
 *
 * Defined by: AI-infra book section 9.3.2 (expert = gate, up and down matrices
 * of 4096 x 1536; expert FLOPs 2*m*P_e) and section 9.4.3 (grouped GEMM over the
 * experts' variable row counts); "Hosting Qwen on Blackwell", section "MoE
 * GEMM" and section "MoE Dispatch - Combine" (combine = weighted accumulation;
 * with expert parallelism a local accumulation over the local experts).
 *
 * For each local expert i and each of its rows r in [offsets[i], offsets[i+1]):
 *   a_r   = MOE_FFN_GATHER ? a[row_token[r],:] : a[r,:]            (length H)
 *   G     = w_gate_up[i, 0..I-1, :]  . a_r   (x s_gate_up[i, 0..I-1] for fp8)
 *   U     = w_gate_up[i, I..2I-1, :] . a_r   (x s_gate_up[i, I..2I-1] for fp8)
 *   h_r   = silu(G) * U  (silu(z) = z / (1 + exp(-z))), fp32, then rounded to
 *           bf16 (round-to-nearest-even) when a_dtype is MOE_BF16
 *   o_r   = w_down[i] . h_r              (x s_down[i, :] for fp8), length H
 *   y != NULL:  y[row_token[r],:] += row_w[r] * o_r   (fp32 atomic adds, so the
 *               order of the k additions to a token is not fixed; with
 *               MOE_FFN_ZERO_Y y is zeroed first on the stream)
 *   y == NULL:  y_perm[r,:] = o_r                     (then call moe_combine)
 * Products accumulate in fp32 (bf16 matrix cores for bf16 and fp8 weights;
 * e4m3 values are exact in bf16).
 *
 * a: [R_cap,H] (or [T,H] with MOE_FFN_GATHER), MOE_BF16 with MOE_BF16 or
 * MOE_FP8_E4M3 weights, or MOE_F32 with MOE_F32 weights.  w_gate_up
 * [E_loc,2I,H] (rows 0..I-1 gate, I..2I-1 up), w_down [E_loc,H,I]; s_gate_up
 * [E_loc,2I] and s_down [E_loc,H] fp32, required for fp8 and ignored otherwise.
 * y [T,H] fp32 or y_perm [R_cap,H] fp32 (exactly one of them non-NULL).
 * workspace: at least moe_ffn_workspace_size(...) bytes, 256-byte aligned.
 * H and I must be multiples of 64; every pointer 16-byte aligned.
 * MOE_FFN_ONLY_GATE_UP / MOE_FFN_ONLY_DOWN split the call into its two halves
 * (same arguments, same workspace, same stream, in that order), e.g. to place
 * other work between them; setting both is MOE_ERR_SHAPE.  MOE_FFN_ZERO_Y is
 * honoured by the call that runs the down half.  MOE_FFN_PACKED_WEIGHTS: both
 * weight tensors come from moe_pack_weights (MOE_ERR_DTYPE with fp32 weights);
 * the results are bit-identical to those with row-major weights.  An unknown
 * flag bit is MOE_ERR_SHAPE.
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_DTYPE, MOE_ERR_WORKSPACE,
 * MOE_ERR_ALIGN, MOE_ERR_HIP.  R_cap == 0 or T == 0 only zeroes y (if asked).
 */
int moe_grouped_ffn(const void *a, int a_dtype, const int32_t *offsets, const int32_t *row_token,
                    const float *row_w, int E_loc, int T, int R_cap, int H, int I,
                    const void *w_gate_up, const void *w_down, int w_dtype,
                    const float *s_gate_up, const float *s_down, float *y, float *y_perm,
                    void *workspace, size_t workspace_bytes, unsigned flags, void *stream);

/* Size of the device scratch array that moe_grouped_ffn_noalloc keeps its intermediate h in. */
#define MOE_NOALLOC_SCRATCH_BYTES (32u << 20)

/*
 * moe_grouped_ffn_noalloc - moe_grouped_ffn without a caller-provided workspace.
 *
 * For callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  Same arguments (less
 * the workspace), same kernels, same results and errors as moe_grouped_ffn; the
 * intermediate h [R_cap, I] lives in a static device array of
 * MOE_NOALLOC_SCRATCH_BYTES (32 MiB) instead.  Each GPU the library runs on holds
 * its own copy of that array from the first call on it until the process ends;
 * the call uses the copy of the current device (``stream`` must belong to it).
 * The call itself allocates nothing (no hipMalloc / hipFree, no allocating
 * library routine).  Limit: moe_ffn_workspace_size(R_cap, E_loc, H, I, a_dtype)
 * must not exceed MOE_NOALLOC_SCRATCH_BYTES (e.g. R_cap * I <= 16 M bf16 values:
 * every decode-sized batch of the 3 x 4096 x 1536 expert with T * k up to 10922),
 * else MOE_ERR_WORKSPACE before anything is enqueued.  Nothing in the array has
 * to start at zero: the gate/up half writes every row of h the down half reads.
 * Every call on one GPU shares its array, which keeps the last call's contents,
 * so calls that overlap on one GPU (several streams, several host threads) race
 * and give wrong results: run them one after another, e.g. on one stream.  With
 * MOE_FFN_ONLY_GATE_UP / MOE_FFN_ONLY_DOWN no other call of this entry point on
 * the same GPU may come between the two halves.
 */
int moe_grouped_ffn_noalloc(const void *a, int a_dtype, const int32_t *offsets, const int32_t *row_token,
                            const float *row_w, int E_loc, int T, int R_cap, int H, int I, const void *w_gate_up,
                            const void *w_down, int w_dtype, const float *s_gate_up, const float *s_down, float *y,
                            float *y_perm, unsigned flags, void *stream);

/*
 * moe_pack_weights - copy expert weights into the packed block layout.
 *
 * Same values, another order in memory; it changes no result.  The
 * expert-parallel layer keeps every local expert's weights resident and reads
 * them all once per call (section "Expert Parallelism" of "Hosting Qwen on
 * Blackwell"; the weight bytes that section 9.3.2 of the AI-infra book counts
 * per expert); the layout only makes that read more sequential: a workgroup
 * that streams 32 weight rows reads one contiguous 32 x 64-value block per
 * 64-wide step of the contraction instead of 32 rows far apart.
 *
 * w: [E, N, K] row-major, MOE_BF16 or MOE_FP8_E4M3 (w_dtype); packed: the same
 * number of bytes, written as, for every group of 32 rows (row = e*N + n over
 * all experts) and every 64-wide K chunk c, the 32 x 64 block of those rows and
 * columns [64c, 64c+64), with the blocks of a row group in order of c and the
 * row groups in order.  fp8 blocks are row-major: element (row, k) is at byte
 *   (row / 32) * 32 * K + (row % 32) * 64 + (k / 64) * 2048 + k % 64.
 * bf16 blocks hold 16-byte pieces (8 values k = 8p .. 8p+7 of the chunk, p = (k % 64) / 8)
 * ordered by p % 4, then p / 4, then block row: element (row, k) is at byte
 *   (row / 32) * 64 * K + (k / 64) * 4096 + (p % 4) * 1024
 *     + ((row % 32) + 32 * (p / 4)) * 16 + (k % 8) * 2,
 * the order in which a wave that streams a block into matrix-core operands
 * reads it, 1 KB contiguously per load.
 * Pass the packed w_gate_up ([E_loc, 2I, H]: N = 2I, K = H) and w_down
 * ([E_loc, H, I]: N = H, K = I) to moe_grouped_ffn or moe_shared_expert (E = 1)
 * with MOE_FFN_PACKED_WEIGHTS; fp8 scales stay as they are.  N a multiple of 32,
 * K of 64; both pointers 16-byte aligned, the buffers must not overlap (the
 * call does not pack in place).  Runs asynchronously on ``stream``.
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE (also for overlapping buffers),
 * MOE_ERR_DTYPE, MOE_ERR_ALIGN, MOE_ERR_HIP.
 */
int moe_pack_weights(const void *w, int w_dtype, int E, int N, int K, void *packed, void *stream);

/*
 * moe_quantize_mx - MXFP8 quantisation of a row-major matrix along its rows.
 *
 * Defined by: "Hosting Qwen on Blackwell", section "Quantization" (the deployed
 * model runs MXFP8: 8-bit E4M3 values sharing a power-of-two scale per block of
 * 32); the block rule below is the reading this library takes of it.
 *
 * For every row r and block b (values v = x[r, 32b .. 32b+31]):
 *   amax = max |v|;  s = amax == 0 ? 0 : clamp(floor(log2 amax) - 8 + 127, 0, 254)
 *   scales[r, b] = s;  codes[r, 32b+i] = E4M3 code nearest to v_i / 2^(s-127),
 *   ties to the even code, magnitudes >= 448 saturate to 448, sign bit kept.
 * x: rows x K, MOE_F32 or MOE_BF16; codes [rows, K] uint8; scales [rows, K/32]
 * uint8.  K must be a multiple of 32 and rows >= 0; x 16-byte aligned, codes
 * 8-byte aligned.  Errors: MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_DTYPE,
 * MOE_ERR_ALIGN, MOE_ERR_HIP.
 */
int moe_quantize_mx(const void *x, int x_dtype, int rows, int K, uint8_t *codes, uint8_t *scales, void *stream);

/* Bytes of workspace moe_grouped_ffn_mx needs (h as MXFP8: R_cap*I codes and R_cap*I/32 scales). */
size_t moe_ffn_mx_workspace_size(int R_cap, int I);

/*
 * moe_grouped_ffn_mx - the SwiGLU expert FFN of moe_grouped_ffn in W8A8 MXFP8.
 *
 * Defined by: the passages of moe_grouped_ffn, with the MXFP8 format of the
 * "Quantization" section of "Hosting Qwen on Blackwell" for activations and
 * weights (weights converted offline, activations quantised on the fly).
 *
 * Same per-row definition as moe_grouped_ffn with every operand an MX tensor:
 * a_r is row r (MOE_FFN_GATHER: row row_token[r]) of the MX activations
 * (a_codes [rows, H], a_scales [rows, H/32], e.g. from moe_quantize_mx);
 * weights wgu_codes [E_loc, 2I, H] + wgu_scales [E_loc, 2I, H/32] and
 * wd_codes [E_loc, H, I] + wd_scales [E_loc, H, I/32].  G and U accumulate
 * exact E4M3 products times their two block scales in fp32 on the fp8 matrix
 * cores; h_r = silu(G) * U in fp32 is quantised per row with the rule of
 * moe_quantize_mx (blocks of 32 along I) into the workspace before the down
 * projection.  Outputs, flags and the combine are those of moe_grouped_ffn;
 * with MOE_FFN_PACKED_WEIGHTS the weight codes are in the packed block layout
 * of moe_pack_weights (packed as MOE_FP8_E4M3 bytes), the scales stay row-major.
 * H and I must be multiples of 128; pointers 16-byte aligned (scale arrays
 * 4-byte aligned); workspace at least moe_ffn_mx_workspace_size(R_cap, I)
 * bytes, 256-byte aligned.  Errors: MOE_ERR_NULL, MOE_ERR_SHAPE,
 * MOE_ERR_DTYPE, MOE_ERR_WORKSPACE, MOE_ERR_ALIGN, MOE_ERR_HIP.
 */
int moe_grouped_ffn_mx(const uint8_t *a_codes, const uint8_t *a_scales, const int32_t *offsets,
                       const int32_t *row_token, const float *row_w, int E_loc, int T, int R_cap, int H, int I,
                       const uint8_t *wgu_codes, const uint8_t *wgu_scales, const uint8_t *wd_codes,
                       const uint8_t *wd_scales, float *y, float *y_perm, void *workspace,
                       size_t workspace_bytes, unsigned flags, void *stream);

/*
 * moe_combine - gate-weighted gather-sum of per-row outputs back to token order.
 *
 * Defined by: "Hosting Qwen on Blackwell", section "MoE Dispatch - Combine"
 * (combine = weighted accumulation); AI-infra book section 9.3.4 (the token's
 * output is the routing-weighted sum of its expert results).
 *
 *   y[t,:] = sum over j = 0..k-1 with token_row[t,j] >= 0 of
 *            topk_w[t,j] * y_perm[token_row[t,j],:]
 * accumulated in fp32 in increasing j (deterministic); y [T,H] is overwritten
 * (rows of tokens without local experts become 0).  y_perm [R_cap,H] fp32,
 * token_row [T,k] int32, topk_w [T,k] fp32.  H a multiple of 4, pointers
 * 16-byte aligned.  Errors: MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_ALIGN, MOE_ERR_HIP.
 */
int moe_combine(const float *y_perm, const int32_t *token_row, const float *topk_w, int T, int k, int H,
                float *y, void *stream);

/*
 * moe_pack_router - the router weight in the layout the decode router reads fastest.
 *
 * For the callers of moe_route_dispatch that keep the router weight resident:
 * out [H/4][E][4] fp32 with out[(j*E + e)*4 + i] = w_router[e, 4j + i], the
 * exact fp32 value of each element (bf16 -> fp32 appends zero bits).  Passed
 * as w_router with w_dtype MOE_F32_ROUTER_PACKED, the logits are the same
 * fused-multiply-add chains on the same values, so routing and gates are
 * bit-identical to the bf16 / fp32 weight; the 64 lanes of a wave (one expert
 * each) then read 1 KB contiguously per load and unpack nothing.  Done once,
 * like loading the weights (it costs E*H*4 bytes of HBM).  w_router [E,H]
 * MOE_BF16 or MOE_F32 (element-aligned); out 16-byte aligned, caller-owned,
 * not overlapping w_router; H a multiple of 4, 1 <= E <= 1024.  Errors:
 * MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_DTYPE, MOE_ERR_ALIGN, MOE_ERR_HIP.
 */
int moe_pack_router(const void *w_router, int w_dtype, int E, int H, float *out, void *stream);

/* Bytes of workspace moe_route_dispatch needs (one ticket counter). */
size_t moe_route_dispatch_workspace_size(void);

/*
 * moe_route_dispatch - moe_route and moe_permute of a decode batch in one launch.
 *
 * Defined by: "Hosting Qwen on Blackwell", section "MoE Dispatch - Combine":
 * for decoding the dispatch work (routing information aggregated, each local
 * expert's tokens grouped for its GEMM) runs as one kernel, where prefill
 * splits it into several because the routing step needs fewer blocks.
 *
 * Results are exactly those of moe_route (topk_ids, topk_w) followed by
 * moe_permute without the x_perm gather (counts, offsets, row_token, row_w,
 * token_row), same layouts and sizes (T = 0 zeroes counts and offsets).  If
 * y_zero is not NULL, y_zero [T,H]
 * fp32 is also zeroed in the same launch (the target of moe_grouped_ffn's
 * fused combine, which then runs without MOE_FFN_ZERO_Y).  Each block routes
 * one token; the last block to finish groups the assignments, so no block
 * ever waits on another.  Supported sizes: 1 <= T <= 512, T*k <= 8192,
 * E <= 256, H a multiple of 8 and at most 16384, x and w_router 16-byte
 * aligned (else MOE_ERR_SHAPE: use moe_route + moe_permute).  The workspace
 * (moe_route_dispatch_workspace_size() bytes, 256-byte aligned) holds a
 * ticket counter that must be zero before the first call (zero it once when
 * allocating); every call leaves it zero.  w_dtype: MOE_BF16, MOE_F32 or
 * MOE_F32_ROUTER_PACKED (w_router written by moe_pack_router, same results).  Calls that share a workspace must
 * not overlap (run them on one stream).  Errors: MOE_ERR_NULL, MOE_ERR_SHAPE,
 * MOE_ERR_DTYPE, MOE_ERR_WORKSPACE, MOE_ERR_ALIGN, MOE_ERR_HIP.
 */
int moe_route_dispatch(const void *x, int x_dtype, const void *w_router, int w_dtype, const float *bias, int T, int H,
                       int E, int k, int e_begin, int e_end, int32_t *topk_ids, float *topk_w, int32_t *counts,
                       int32_t *offsets, int32_t *row_token, float *row_w, int32_t *token_row, float *y_zero,
                       void *workspace, size_t workspace_bytes, void *stream);

/*
 * Bytes of workspace moe_decode_layer needs: 256-byte aligned control words (one per local expert
 * plus a few), then h [E_loc, T, I] bf16.
 */
size_t moe_decode_layer_workspace_size(int T, int k, int E_loc, int I);

/*
 * moe_decode_layer - the whole MoE layer of a decode batch in one launch.
 *
 * Defined by: "Hosting Qwen on Blackwell", section "Expert parallelism" (for decoding the whole
 * MoE kernel is merged into one), with the steps of moe_route, moe_permute and moe_grouped_ffn
 * (fused combine) as defined above.
 *
 * Results: topk_ids, topk_w exactly as moe_route; counts, offsets, row_token, row_w, token_row
 * exactly as moe_permute (no x_perm); y [T,H] fp32 OVERWRITTEN with the layer output
 *   y[t,:] = sum over the local assignments (t, j) of topk_w[t,j] * FFN_{topk_ids[t,j]}(x[t,:])
 * with the FFN of moe_grouped_ffn (h rounded to bf16; fp32 atomic accumulation, so the order of a
 * token's additions is not fixed).  One persistent launch: routing items, then gate/up items, then
 * down items, taken from a work queue by at most as many workgroups as the device holds at once.
 * The gate/up items wait for the grouping and compute h for the routed rows only; h [E_loc, T, I]
 * (row = token) is left in the workspace after the control words, and its rows of the routed
 * (token, expert) pairs are bit-identical to moe_grouped_ffn's h with few rows per expert (the
 * other rows are not written).
 *
 * x [T,H] MOE_BF16; w_router [E,H] MOE_BF16 or MOE_F32, or MOE_F32_ROUTER_PACKED (moe_pack_router);
 * bias [E] or NULL; expert weights and scales as moe_grouped_ffn (MOE_BF16 or MOE_FP8_E4M3; flag
 * MOE_FFN_PACKED_WEIGHTS for weights from moe_pack_weights; no other flag).  Supported sizes:
 * 0 <= T <= 64 (decode batches; larger ones use moe_route_dispatch or moe_route + moe_permute, then
 * moe_grouped_ffn), 1 <= k <= min(E, 32), E <= 256, H and I multiples of 64, H <= 16384; T == 0
 * only zeroes counts and offsets.  Pointers 16-byte aligned.
 * The workspace (moe_decode_layer_workspace_size bytes, 256-byte aligned) must be all zero before
 * the first call (zero it once when allocating); every call leaves its control words zero again.
 * Calls that share a workspace must not overlap (run them on one stream).  Its uint32 word 4
 * (byte 16) is a diagnostic: nonzero if a wait inside the kernel gave up (never expected; the
 * results of that call are then invalid); the library does not clear it.
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_DTYPE, MOE_ERR_WORKSPACE, MOE_ERR_ALIGN, MOE_ERR_HIP.
 */
int moe_decode_layer(const void *x, int x_dtype, const void *w_router, int wr_dtype, const float *bias, int T, int H,
                     int E, int k, int e_begin, int e_end, int I, const void *w_gate_up, const void *w_down,
                     int w_dtype, const float *s_gate_up, const float *s_down, int32_t *topk_ids, float *topk_w,
                     int32_t *counts, int32_t *offsets, int32_t *row_token, float *row_w, int32_t *token_row,
                     float *y, void *workspace, size_t workspace_bytes, unsigned flags, void *stream);

/* Bytes of workspace moe_shared_expert needs (h [T, I_s] of x_dtype, then its row maps). */
size_t moe_shared_workspace_size(int T, int I_s, int x_dtype);

/*
 * moe_shared_expert - an always-active (shared) expert added to the layer output.
 *
 * Defined by: "PagedAttention, speculative decoding, MoE and Blackwell", MoE
 * list, the bullet on shared experts: besides the routed experts a model may
 * keep a few experts that process every token.  Reading taken: each shared
 * expert is a SwiGLU FFN of the routed experts' form and its output is added
 * to the token's output with weight 1 (no gate); several shared experts are
 * one FFN whose intermediate is their intermediates side by side (the sum of
 * SwiGLU FFNs equals that FFN exactly).
 *
 *   y[t,:] += W_d h_t,  h_t = silu(W_g x_t) * (W_u x_t)   for every t < T
 * with x [T,H] (bf16 or fp32), w_gate_up [2*I_s, H] (rows 0..I_s-1 gate,
 * I_s..2*I_s-1 up), w_down [H, I_s], element types and fp8 scales
 * (s_gate_up [2*I_s], s_down [H]) as in moe_grouped_ffn, and h rounded to bf16
 * for bf16 activations.  y [T,H] fp32 accumulates: call it after
 * moe_grouped_ffn's fused combine or moe_combine on the same stream, or pass
 * MOE_FFN_ZERO_Y for the shared expert alone; MOE_FFN_PACKED_WEIGHTS (bf16 and
 * fp8 weights) reads weights packed by moe_pack_weights with E = 1; any other
 * flag bit is MOE_ERR_SHAPE.  For T > 128
 * each element of y receives one fp32 add; for T <= 128 (bf16 activations)
 * the contraction is split over many workgroups to keep HBM busy, so G, U and
 * y receive several fp32 adds of partial sums in no fixed order (run-to-run
 * rounding differences).  H and I_s multiples of 64; pointers 16-byte
 * aligned, workspace at least moe_shared_workspace_size(T, I_s, x_dtype)
 * bytes, 256-byte aligned.  Errors: MOE_ERR_NULL, MOE_ERR_SHAPE,
 * MOE_ERR_DTYPE, MOE_ERR_WORKSPACE, MOE_ERR_ALIGN, MOE_ERR_HIP.
 */
int moe_shared_expert(const void *x, int x_dtype, int T, int H, int I_s, const void *w_gate_up, const void *w_down,
                      int w_dtype, const float *s_gate_up, const float *s_down, float *y, void *workspace,
                      size_t workspace_bytes, unsigned flags, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */

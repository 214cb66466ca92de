/*
 * CPU oracle for the Mixture-of-Experts FFN layer.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously correct
 * definition that the GPU path is checked against.  Only the test suite, the
 * package smoke check and the benchmark's CPU-baseline leg may load it; the
 * GPU library never links, calls or includes anything from here, and this
 * file includes nothing from the GPU library.
 *
 * What it computes (sources are the three pages the method is taken from):
 *   - "AI-infra book, ch. 9", section 9.3.4 (Fig. 9-16): a router picks k
 *     experts per token, rows are grouped by expert, every expert runs its
 *     FFN on its rows, and the token's output is the routing-weighted sum of
 *     its k expert outputs.
 *   - "PagedAttention, speculative decoding, MoE and Blackwell", MoE bullet
 *     list: a learned gating network sends each token to its top-K experts.
 *   - "Hosting Qwen on Blackwell", section "MoE Dispatch - Combine": dispatch
 *     groups the tokens of each expert into GEMM input buffers; combine is a
 *     weighted accumulation; with replicated inputs (section "Expert
 *     parallelism") a rank keeps only the tokens routed to its own experts.
 *   - Book, section 9.3.2: the Qwen3-235B-A22B expert is three matrices of
 *     4096 x 1536 (gate, up, down); the FFN form is SwiGLU.
 *
 * Readings where the pages are silent (each is data, not an optimisation):
 *   R1 router logit = fp32 fused-multiply-add chain over h = 0..H-1 in
 *      ascending order, starting at +0, then one fp32 add of the bias;
 *   R2 top-k order = logit descending, ties (IEEE equality, so -0 == +0) to
 *      the lower expert index;
 *   R3 gates = softmax over the k selected logits (fp64), which equals a full
 *      softmax renormalised over the selected experts;
 *   R4 a rank that owns experts [e_begin, e_end) drops the other assignments
 *      from its combine and does not renormalise the remaining gates;
 *   R5 expert FFN: G = Wg x, U = Wu x, h = silu(G) * U, o = Wd h; for bf16
 *      models h is rounded fp64 -> fp32 -> bf16 (RNE) before the down
 *      projection (the precision the GPU feeds to it), for fp32 models only
 *      fp64 -> fp32; fp8 weights are exact e4m3 values times a fp32 scale of
 *      their output channel;
 *   R6 output y[t] = sum over kept j of gate_j * o_j, accumulated in fp64 and
 *      stored fp32;
 *   R7 permuted rows are ordered by (expert ascending, token ascending).
 *   R8 MXFP8 (the OCP microscaling format the "Quantization" section of
 *      "Hosting Qwen on Blackwell" deploys): every 32 consecutive values along
 *      the contraction axis share one E8M0 scale 2^(s-127); with amax the
 *      block's largest magnitude, s = clamp(floor(log2 amax) - 8 + 127, 0, 254)
 *      (8 = exponent of the largest e4m3 power of two), s = 0 for an all-zero
 *      block; each value becomes the e4m3 code nearest to v / 2^(s-127),
 *      ties to the even code, magnitudes above 448 saturate to 448, the sign
 *      bit is kept.  In the W8A8 layer x is quantised per token row, h from
 *      its fp32 value per row, and the weights arrive already quantised.
 *   R10 a shared expert ("PagedAttention, speculative decoding, MoE and
 *      Blackwell", MoE list, shared-experts bullet) is an FFN of the R5 form
 *      that every token passes through; its output is added to the token's
 *      output with weight 1, and several shared experts are one FFN whose
 *      intermediate is theirs side by side.
 *
 * Everything else accumulates in fp64 over the exact stored input values.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ODT_F32 = 0, ODT_BF16 = 1, ODT_E4M3 = 2 };

/* ---- storage decoding ---------------------------------------------------- */

static float bf16_bits_to_float(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* OCP 8-bit E4M3 ("fn"): 1 sign, 4 exponent (bias 7), 3 mantissa bits; no
 * infinities; exponent 0 is subnormal (m/8 * 2^-6); 0x7F and 0xFF are NaN. */
double oracle_e4m3_value(uint8_t code)
{
    int s = code >> 7, e = (code >> 3) & 15, m = code & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m / 8.0, -6);
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -v : v;
}

/* float -> bf16, round to nearest, ties to even (finite inputs). */
uint16_t oracle_bf16_round(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    uint32_t lsb = (u >> 16) & 1u;
    return (uint16_t)((u + 0x7FFFu + lsb) >> 16);
}

/* R8: value -> e4m3 code, round to nearest, ties to the even code, saturating at 448,
 * sign bit kept.  The positive codes 0x00..0x7E are ordered by value, so the nearest
 * code is found by bisection over their exact values. */
uint8_t oracle_e4m3_encode(double v)
{
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs(v);
    if (a >= oracle_e4m3_value(126))
        return sign | 126;
    int lo = 0, hi = 126; /* value(lo) <= a < value(hi) */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (oracle_e4m3_value((uint8_t)mid) <= a)
            lo = mid;
        else
            hi = mid;
    }
    double dl = a - oracle_e4m3_value((uint8_t)lo), dh = oracle_e4m3_value((uint8_t)hi) - a;
    int c = dl < dh ? lo : (dh < dl ? hi : ((lo & 1) ? hi : lo));
    return sign | (uint8_t)c;
}

/* R8: E8M0 scale byte of a block with largest magnitude amax. */
uint8_t oracle_mx_scale(double amax)
{
    if (amax == 0.0)
        return 0;
    int ex;
    frexp(amax, &ex); /* amax = f * 2^ex, f in [0.5, 1): floor(log2 amax) = ex - 1 */
    int s = ex - 1 - 8 + 127;
    return (uint8_t)(s < 0 ? 0 : (s > 254 ? 254 : s));
}

/* R8: one block of n (<= 32) values -> codes and its scale byte. */
static uint8_t mx_block(const double *v, int n, uint8_t *codes)
{
    double amax = 0.0;
    for (int i = 0; i < n; i++)
        amax = fmax(amax, fabs(v[i]));
    uint8_t s = oracle_mx_scale(amax);
    for (int i = 0; i < n; i++)
        codes[i] = oracle_e4m3_encode(ldexp(v[i], 127 - (int)s));
    return s;
}

static double elem(const void *p, int dt, size_t i);

/* R8: rows x K values (f32 or bf16) -> codes [rows, K], scales [rows, K/32]; K % 32 == 0. */
void oracle_mx_quantize(const void *x, int x_dt, int rows, int K, uint8_t *codes, uint8_t *scales)
{
#pragma omp parallel for schedule(static)
    for (int r = 0; r < rows; r++) {
        double v[32];
        for (int b = 0; b < K / 32; b++) {
            for (int i = 0; i < 32; i++)
                v[i] = elem(x, x_dt, (size_t)r * K + 32 * b + i);
            scales[(size_t)r * (K / 32) + b] = mx_block(v, 32, codes + (size_t)r * K + 32 * b);
        }
    }
}

/* The 256 e4m3 values, filled once from oracle_e4m3_value (call it outside parallel regions). */
static double e4m3_tab[256];
static int e4m3_tab_ready = 0;

static const double *e4m3_table(void)
{
    if (!e4m3_tab_ready) {
        for (int c = 0; c < 256; c++)
            e4m3_tab[c] = oracle_e4m3_value((uint8_t)c);
        e4m3_tab_ready = 1;
    }
    return e4m3_tab;
}

/* Dot product of an exact fp64 vector a[0..K-1] with MX row ``row`` (codes [.., K], scales
 * [.., K/32]): element i of the row is code * 2^(scale of its block - 127), formed exactly (the
 * product of an e4m3 value and a power of two in [2^-127, 2^127] is exact in fp64), and the
 * products are summed for i ascending. */
static double mx_row_dot(const double *a, const uint8_t *codes, const uint8_t *scales, size_t row, int K,
                         const double *tab)
{
    const uint8_t *q = codes + row * (size_t)K;
    const uint8_t *sc = scales + row * (size_t)(K / 32);
    double acc = 0.0;
    for (int b = 0; b < K / 32; b++) {
        const double f = ldexp(1.0, (int)sc[b] - 127);
        for (int i = 32 * b; i < 32 * b + 32; i++)
            acc += a[i] * (tab[q[i]] * f);
    }
    return acc;
}

static double elem(const void *p, int dt, size_t i)
{
    switch (dt) {
    case ODT_F32: return (double)((const float *)p)[i];
    case ODT_BF16: return (double)bf16_bits_to_float(((const uint16_t *)p)[i]);
    default: return oracle_e4m3_value(((const uint8_t *)p)[i]);
    }
}

static float elem_f32(const void *p, int dt, size_t i)
{
    return dt == ODT_F32 ? ((const float *)p)[i] : bf16_bits_to_float(((const uint16_t *)p)[i]);
}

/* ---- routing ------------------------------------------------------------- */

/* R1: logits[t,e] for all t, e (x [T,H], w [E,H], bias [E] or NULL). */
void oracle_router_logits(const void *x, int x_dt, const void *w, int w_dt, const float *bias,
                          int T, int H, int E, float *logits)
{
#pragma omp parallel for schedule(dynamic, 4)
    for (int t = 0; t < T; t++) {
        for (int e = 0; e < E; e++) {
            float acc = 0.0f;
            for (int h = 0; h < H; h++)
                acc = fmaf(elem_f32(x, x_dt, (size_t)t * H + h), elem_f32(w, w_dt, (size_t)e * H + h), acc);
            if (bias)
                acc = acc + bias[e];
            logits[(size_t)t * E + e] = acc;
        }
    }
}

/* R2 + R3 for one token: pick k experts by (logit desc, index asc), then the
 * gates.  ``taken`` is scratch of E bytes. */
static void topk_one(const float *l, int E, int k, int32_t *ids, float *gates, unsigned char *taken)
{
    memset(taken, 0, (size_t)E);
    for (int j = 0; j < k; j++) {
        int best = -1;
        for (int e = 0; e < E; e++) {
            if (taken[e])
                continue;
            /* strictly greater wins; equal logits keep the lower index found first */
            if (best < 0 || l[e] > l[best])
                best = e;
        }
        taken[best] = 1;
        ids[j] = best;
    }
    double m = (double)l[ids[0]], sum = 0.0, u[64];
    for (int j = 0; j < k; j++) {
        u[j] = exp((double)l[ids[j]] - m);
        sum += u[j];
    }
    for (int j = 0; j < k; j++)
        gates[j] = (float)(u[j] / sum);
}

/* Top-k and gates from given logits [T,E]; k <= 64. */
int oracle_topk(const float *logits, int T, int E, int k, int32_t *topk_ids, float *topk_w)
{
    if (k < 1 || k > 64 || k > E)
        return -1;
#pragma omp parallel
    {
        unsigned char *taken = (unsigned char *)malloc((size_t)E);
#pragma omp for schedule(static)
        for (int t = 0; t < T; t++)
            topk_one(logits + (size_t)t * E, E, k, topk_ids + (size_t)t * k, topk_w + (size_t)t * k, taken);
        free(taken);
    }
    return 0;
}

/* Router + top-k + gates.  ``logits`` [T,E] is an output (may not be NULL). */
int oracle_route(const void *x, int x_dt, const void *w, int w_dt, const float *bias,
                 int T, int H, int E, int k, int32_t *topk_ids, float *topk_w, float *logits)
{
    oracle_router_logits(x, x_dt, w, w_dt, bias, T, H, E, logits);
    return oracle_topk(logits, T, E, k, topk_ids, topk_w);
}

/* ---- dispatch (permutation) ---------------------------------------------- */

/* R7: stable counting sort of the local assignments by expert.
 * counts [e_end-e_begin], offsets [e_end-e_begin+1], row_token/row_w [R],
 * token_row [T,k] (-1 for assignments to non-local experts).  Returns R. */
int oracle_permute(const int32_t *topk_ids, const float *topk_w, int T, int k, int e_begin, int e_end,
                   int32_t *counts, int32_t *offsets, int32_t *row_token, float *row_w, int32_t *token_row)
{
    int El = e_end - e_begin;
    for (int i = 0; i < El; i++)
        counts[i] = 0;
    for (size_t a = 0; a < (size_t)T * k; a++) {
        int e = topk_ids[a];
        if (e >= e_begin && e < e_end)
            counts[e - e_begin]++;
    }
    offsets[0] = 0;
    for (int i = 0; i < El; i++)
        offsets[i + 1] = offsets[i] + counts[i];
    int32_t *cursor = (int32_t *)malloc(sizeof(int32_t) * (size_t)(El > 0 ? El : 1));
    for (int i = 0; i < El; i++)
        cursor[i] = offsets[i];
    for (int t = 0; t < T; t++) {
        for (int j = 0; j < k; j++) {
            size_t a = (size_t)t * k + j;
            int e = topk_ids[a];
            if (e >= e_begin && e < e_end) {
                int r = cursor[e - e_begin]++;
                row_token[r] = t;
                row_w[r] = topk_w[a];
                token_row[a] = r;
            } else {
                token_row[a] = -1;
            }
        }
    }
    free(cursor);
    return offsets[El];
}

/* ---- expert FFN and combine ---------------------------------------------- */

/* R5 + R6, token-major: y for the listed tokens only (y_out [n_tok, H]).
 * w_gate_up [E_loc, 2I, H] (rows 0..I-1 gate, I..2I-1 up), w_down [E_loc, H, I];
 * s_gate_up [E_loc, 2I], s_down [E_loc, H] are per-output-channel scales used
 * only when w_dt is e4m3.  round_h: 1 = h goes fp64 -> fp32 -> bf16, 0 = fp64 -> fp32. */
void oracle_layer_tokens(const int32_t *tokens, int n_tok, const void *x, int x_dt,
                         const int32_t *topk_ids, const float *topk_w, int T, int H, int k,
                         int e_begin, int e_end, int I, const void *w_gate_up, const void *w_down, int w_dt,
                         const float *s_gate_up, const float *s_down, int round_h, float *y_out)
{
    (void)T;
#pragma omp parallel
    {
        double *yacc = (double *)malloc(sizeof(double) * (size_t)H);
        double *xt = (double *)malloc(sizeof(double) * (size_t)H);
        double *hb = (double *)malloc(sizeof(double) * (size_t)I);
#pragma omp for schedule(dynamic, 1)
        for (int q = 0; q < n_tok; q++) {
            int t = tokens[q];
            for (int n = 0; n < H; n++) {
                yacc[n] = 0.0;
                xt[n] = elem(x, x_dt, (size_t)t * H + n);
            }
            for (int j = 0; j < k; j++) {
                int e = topk_ids[(size_t)t * k + j];
                if (e < e_begin || e >= e_end)
                    continue; /* R4 */
                size_t le = (size_t)(e - e_begin);
                double g = (double)topk_w[(size_t)t * k + j];
                for (int i = 0; i < I; i++) {
                    double G = 0.0, U = 0.0;
                    size_t rg = (le * 2 * I + i) * (size_t)H, ru = (le * 2 * I + I + i) * (size_t)H;
                    for (int h = 0; h < H; h++) {
                        G += xt[h] * elem(w_gate_up, w_dt, rg + h);
                        U += xt[h] * elem(w_gate_up, w_dt, ru + h);
                    }
                    if (w_dt == ODT_E4M3) {
                        G *= (double)s_gate_up[le * 2 * I + i];
                        U *= (double)s_gate_up[le * 2 * I + I + i];
                    }
                    double hv = G / (1.0 + exp(-G)) * U;
                    float hf = (float)hv;
                    hb[i] = round_h ? (double)bf16_bits_to_float(oracle_bf16_round(hf)) : (double)hf;
                }
                for (int n = 0; n < H; n++) {
                    double o = 0.0;
                    size_t rd = (le * H + n) * (size_t)I;
                    for (int i = 0; i < I; i++)
                        o += hb[i] * elem(w_down, w_dt, rd + i);
                    if (w_dt == ODT_E4M3)
                        o *= (double)s_down[le * H + n];
                    yacc[n] += g * o;
                }
            }
            for (int n = 0; n < H; n++)
                y_out[(size_t)q * H + n] = (float)yacc[n];
        }
        free(yacc);
        free(xt);
        free(hb);
    }
}

/* R5 + R6 + R8, token-major, W8A8 MXFP8: x is quantised per token row, each selected
 * local expert runs on the quantised row with MX weights (codes [E_loc, 2I, H] and
 * [E_loc, H, I], scales [E_loc, 2I, H/32] and [E_loc, H, I/32]); h is computed in fp64,
 * rounded to fp32 and quantised per row (blocks of 32 along I) before the down projection. */
void oracle_layer_tokens_mx(const int32_t *tokens, int n_tok, const void *x, int x_dt,
                            const int32_t *topk_ids, const float *topk_w, int H, int k,
                            int e_begin, int e_end, int I, const uint8_t *wgu_q, const uint8_t *wgu_s,
                            const uint8_t *wd_q, const uint8_t *wd_s, float *y_out)
{
    const double *tab = e4m3_table();
#pragma omp parallel
    {
        double *yacc = (double *)malloc(sizeof(double) * (size_t)H);
        double *xv = (double *)malloc(sizeof(double) * (size_t)H);
        double *xq = (double *)malloc(sizeof(double) * (size_t)H);
        double *hv = (double *)malloc(sizeof(double) * (size_t)I);
        double *hq = (double *)malloc(sizeof(double) * (size_t)I);
        uint8_t codes[32];
#pragma omp for schedule(dynamic, 1)
        for (int q = 0; q < n_tok; q++) {
            int t = tokens[q];
            for (int n = 0; n < H; n++) {
                yacc[n] = 0.0;
                xv[n] = elem(x, x_dt, (size_t)t * H + n);
            }
            for (int b = 0; b < H / 32; b++) {
                uint8_t sb = mx_block(xv + 32 * b, 32, codes);
                for (int i = 0; i < 32; i++)
                    xq[32 * b + i] = ldexp(oracle_e4m3_value(codes[i]), (int)sb - 127);
            }
            for (int j = 0; j < k; j++) {
                int e = topk_ids[(size_t)t * k + j];
                if (e < e_begin || e >= e_end)
                    continue; /* R4 */
                size_t le = (size_t)(e - e_begin);
                double g = (double)topk_w[(size_t)t * k + j];
                for (int i = 0; i < I; i++) {
                    double G = mx_row_dot(xq, wgu_q, wgu_s, le * 2 * I + i, H, tab);
                    double U = mx_row_dot(xq, wgu_q, wgu_s, le * 2 * I + I + i, H, tab);
                    hv[i] = (double)(float)(G / (1.0 + exp(-G)) * U);
                }
                for (int b = 0; b < I / 32; b++) {
                    uint8_t sb = mx_block(hv + 32 * b, 32, codes);
                    for (int i = 0; i < 32; i++)
                        hq[32 * b + i] = ldexp(oracle_e4m3_value(codes[i]), (int)sb - 127);
                }
                for (int n = 0; n < H; n++)
                    yacc[n] += g * mx_row_dot(hq, wd_q, wd_s, le * H + n, I, tab);
            }
            for (int n = 0; n < H; n++)
                y_out[(size_t)q * H + n] = (float)yacc[n];
        }
        free(yacc);
        free(xv);
        free(xq);
        free(hv);
        free(hq);
    }
}

/* R5 + R8, per assignment row: the MXFP8 intermediate of row r (token row_token[r], local
 * expert row_expert[r]), exactly as oracle_layer_tokens_mx forms it before the down
 * projection: h_codes [R, I], h_scales [R, I/32]. */
void oracle_h_mx(const int32_t *row_token, const int32_t *row_expert, int R, const void *x, int x_dt, int H, int I,
                 const uint8_t *wgu_q, const uint8_t *wgu_s, uint8_t *h_codes, uint8_t *h_scales)
{
    const double *tab = e4m3_table();
#pragma omp parallel
    {
        double *xq = (double *)malloc(sizeof(double) * (size_t)H);
        double *xv = (double *)malloc(sizeof(double) * (size_t)H);
        double *hv = (double *)malloc(sizeof(double) * (size_t)I);
        uint8_t codes[32];
#pragma omp for schedule(dynamic, 4)
        for (int r = 0; r < R; r++) {
            int t = row_token[r];
            size_t le = (size_t)row_expert[r];
            for (int n = 0; n < H; n++)
                xv[n] = elem(x, x_dt, (size_t)t * H + n);
            for (int b = 0; b < H / 32; b++) {
                uint8_t sb = mx_block(xv + 32 * b, 32, codes);
                for (int i = 0; i < 32; i++)
                    xq[32 * b + i] = ldexp(oracle_e4m3_value(codes[i]), (int)sb - 127);
            }
            for (int i = 0; i < I; i++) {
                double G = mx_row_dot(xq, wgu_q, wgu_s, le * 2 * I + i, H, tab);
                double U = mx_row_dot(xq, wgu_q, wgu_s, le * 2 * I + I + i, H, tab);
                hv[i] = (double)(float)(G / (1.0 + exp(-G)) * U);
            }
            for (int b = 0; b < I / 32; b++)
                h_scales[(size_t)r * (I / 32) + b] = mx_block(hv + 32 * b, 32, h_codes + (size_t)r * I + 32 * b);
        }
        free(xq);
        free(xv);
        free(hv);
    }
}

/* R10 (with R5's h rounding), token-major: the shared expert's contribution
 * W_d (silu(W_g x_t) * (W_u x_t)) for the listed tokens (y_out [n_tok, H], fp64
 * stored fp32).  w_gate_up [2*I_s, H] (rows 0..I_s-1 gate), w_down [H, I_s];
 * s_gate_up [2*I_s], s_down [H] per-output-channel scales for e4m3 weights. */
void oracle_shared_tokens(const int32_t *tokens, int n_tok, const void *x, int x_dt, int H, int I_s,
                          const void *w_gate_up, const void *w_down, int w_dt, const float *s_gate_up,
                          const float *s_down, int round_h, float *y_out)
{
#pragma omp parallel
    {
        double *xt = (double *)malloc(sizeof(double) * (size_t)H);
        double *hb = (double *)malloc(sizeof(double) * (size_t)I_s);
#pragma omp for schedule(dynamic, 1)
        for (int q = 0; q < n_tok; q++) {
            int t = tokens[q];
            for (int n = 0; n < H; n++)
                xt[n] = elem(x, x_dt, (size_t)t * H + n);
            for (int i = 0; i < I_s; i++) {
                double G = 0.0, U = 0.0;
                size_t rg = (size_t)i * H, ru = (size_t)(I_s + i) * H;
                for (int h = 0; h < H; h++) {
                    G += xt[h] * elem(w_gate_up, w_dt, rg + h);
                    U += xt[h] * elem(w_gate_up, w_dt, ru + h);
                }
                if (w_dt == ODT_E4M3) {
                    G *= (double)s_gate_up[i];
                    U *= (double)s_gate_up[I_s + i];
                }
                float hf = (float)(G / (1.0 + exp(-G)) * U);
                hb[i] = round_h ? (double)bf16_bits_to_float(oracle_bf16_round(hf)) : (double)hf;
            }
            for (int n = 0; n < H; n++) {
                double o = 0.0;
                for (int i = 0; i < I_s; i++)
                    o += hb[i] * elem(w_down, w_dt, (size_t)n * I_s + i);
                if (w_dt == ODT_E4M3)
                    o *= (double)s_down[n];
                y_out[(size_t)q * H + n] = (float)o;
            }
        }
        free(xt);
        free(hb);
    }
}

/* Combine of unweighted per-row expert outputs y_perm [R, H]:
 * y[t] = sum_{j : token_row[t,j] >= 0} topk_w[t,j] * y_perm[token_row[t,j]] (fp64, stored fp32). */
void oracle_combine(const float *y_perm, const int32_t *token_row, const float *topk_w, int T, int k, int H, float *y)
{
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; t++) {
        for (int n = 0; n < H; n++) {
            double acc = 0.0;
            for (int j = 0; j < k; j++) {
                int r = token_row[(size_t)t * k + j];
                if (r >= 0)
                    acc += (double)topk_w[(size_t)t * k + j] * (double)y_perm[(size_t)r * H + n];
            }
            y[(size_t)t * H + n] = (float)acc;
        }
    }
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * moe_oracle.c -- plain, slow, obviously-correct CPU oracle for the W4A16
 * Mixture-of-Experts expert layer.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library. The GPU product path
 * never calls it and shares no code, header, table or helper with it.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fPIC -shared (no -ffast-math, so
 * x87/SSE flush-to-zero and denormals-are-zero stay off and a*b+c is never
 * fused behind our back).
 *
 * Pages followed (cited by title and section):
 *   [FI]  "FlashInfer, CuTe DSL W4A16 MoE optimization and bitwise-exactness
 *         tests" (FlashInfer PR #7196 analysis): section 1 (`moe_finalize.py`,
 *         fp32 multiply for the first slot, then fp32 FMA without FTZ in slot
 *         order); section 2 (SwiGLU, combine order); section 3 (shared exact
 *         reference: bf16 weight decode, scale layout, controlled GEMM,
 *         activation, ordered combine).
 *   [IL]  "T2-1-3 Qwen3-MoE inference optimization report" (InfiniLM PR #500):
 *         section 2.2 (bucket routing ids into per-expert counts and a
 *         permutation; gather; grouped GEMMs gate/up/down + SwiGLU; weight
 *         the rows and scatter them back to tokens).
 *   [GC]  "GC-MoE: Overlapping Expert-Parallel Token Dispatch with FP8/FP4
 *         Grouped GEMM via CUDA Green Contexts" (abstract): expert-parallel
 *         layers, fused SwiGLU, optional (fused) shared experts.
 *
 * Readings of points the pages leave open (each also listed in the design
 * notes): int4 weights are two's-complement nibbles, element k of a row in
 * byte k/2, even k in the low nibble, rows K-contiguous, one bf16 scale per
 * (row, 128-wide K group), no zero point; w13 rows [0, I) are gate and
 * [I, 2I) are up; silu(z) = z / (1 + exp(-z)); h, y and the layer output are
 * rounded to bf16 once each; the top-k order is (logit desc, index asc).
 * Shared experts ([GC] names them without defining them): S always-on experts
 * with the routed experts' shape, applied to every token; each one's bf16
 * output is added to the binary32 combine with weight 1, after the routed
 * slots, in shared-expert order (the first term of a token with no present
 * routed slot initialises the accumulator).
 *
 * Arithmetic: every dot product is an fp64 sum in ascending k (products of a
 * bf16 activation and an exact dequantised weight are exact in fp64), then a
 * single round-to-nearest-even to the stored type. The combine is IEEE
 * binary32 multiply / fusedMultiplyAdd exactly as the pages fix it.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------ */
/* number formats                                                      */
/* ------------------------------------------------------------------ */

/* bf16 bit pattern -> value (bf16 is the top half of a binary32). */
static double bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static uint32_t f32_bits(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return u;
}

/*
 * double -> bf16 with ONE round-to-nearest-even. bf16 has 8 significant bits
 * and binary32's exponent range: normal quantum 2^(e-7) for 2^e <= |d| <
 * 2^(e+1), subnormal quantum 2^-133 below 2^-126, overflow to infinity once
 * the rounded value reaches 2^128. Scaling by powers of two is exact in fp64
 * for every value that reaches here, and nearbyint() rounds half to even in
 * the default rounding mode.
 */
uint16_t oracle_bf16_from_double(double d)
{
    uint16_t sign = signbit(d) ? 0x8000u : 0u;
    if (isnan(d))
        return (uint16_t)(sign | 0x7FC0u);
    double a = fabs(d);
    if (a == 0.0)
        return sign;
    if (isinf(a) || a >= 0x1p128)
        return (uint16_t)(sign | 0x7F80u);
    int e;
    (void)frexp(a, &e); /* a = m * 2^e, m in [0.5, 1): 2^(e-1) <= a < 2^e */
    int qexp = (e - 1 < -126) ? -133 : (e - 1) - 7;
    double r = nearbyint(ldexp(a, -qexp)) ;
    double v = ldexp(r, qexp);
    if (v >= 0x1p128)
        return (uint16_t)(sign | 0x7F80u);
    float f = (float)v; /* exact: v is a bf16 value */
    return (uint16_t)(sign | ((f32_bits(f) >> 16) & 0x7FFFu));
}

/* The stored int4 code of weight element (n, k) of expert e, as a signed int. */
static int int4_code(const uint8_t *wq, int64_t N, int64_t K, int64_t e, int64_t n, int64_t k)
{
    uint8_t byte = wq[(e * N + n) * (K / 2) + k / 2];
    int nib = (k & 1) ? (byte >> 4) : (byte & 0x0F);
    return nib >= 8 ? nib - 16 : nib;
}

/* Dequantised weight W[e][n][k] = q * s[e][n][k / G]; exact in fp64. */
static double weight(const uint8_t *wq, const uint16_t *s, int64_t N, int64_t K, int64_t G,
                     int64_t e, int64_t n, int64_t k)
{
    return (double)int4_code(wq, N, K, e, n, k) * bf16_to_double(s[(e * N + n) * (K / G) + k / G]);
}

static double silu(double z) { return z / (1.0 + exp(-z)); }

void oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int oracle_get_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------ */
/* step 1: routing                                                     */
/* ------------------------------------------------------------------ */

/*
 * Top-k routing of T tokens over E experts (row-major logits [T][E]).
 * Selection order: larger logit first, lower expert index first among equal
 * logits (IEEE equality, so -0 == +0). The i-th selected expert is slot i.
 * Weight of slot i: softmax over all E logits, keep the k selected
 * probabilities, renormalise them to sum to one; done in fp64, rounded once
 * to binary32.
 */
void oracle_route(int T, int E, int k, const float *logits, int32_t *topk_ids, float *topk_w)
{
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        const float *l = logits + (int64_t)t * E;
        char *taken = (char *)calloc((size_t)E, 1);
        double *p = (double *)malloc(sizeof(double) * (size_t)E);
        int32_t *ids = topk_ids + (int64_t)t * k;
        for (int j = 0; j < k; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                if (taken[e])
                    continue;
                if (best < 0 || l[e] > l[best])
                    best = e;
            }
            taken[best] = 1;
            ids[j] = best;
        }
        /* softmax over all experts (shifted by the max for range safety) */
        double m = (double)l[ids[0]];
        double z = 0.0;
        for (int e = 0; e < E; ++e) {
            p[e] = exp((double)l[e] - m);
            z += p[e];
        }
        for (int e = 0; e < E; ++e)
            p[e] /= z;
        double keep = 0.0;
        for (int j = 0; j < k; ++j)
            keep += p[ids[j]];
        for (int j = 0; j < k; ++j)
            topk_w[(int64_t)t * k + j] = (float)(p[ids[j]] / keep);
        free(p);
        free(taken);
    }
}

/* ------------------------------------------------------------------ */
/* step 2: permutation                                                 */
/* ------------------------------------------------------------------ */

/*
 * Bucket the T*k routed slots by local expert (experts [begin, begin+E_loc)).
 * counts[e] = slots routed to local expert e; offsets = exclusive scan
 * (E_loc+1 entries); slots are placed token-ascending within each expert
 * segment: row r holds slot id t*k+j in perm[r], inv_perm[t*k+j] = r.
 * Non-local slots get inv_perm -1; perm entries at r >= R are -1.
 */
void oracle_permute(int T, int k, int expert_begin, int E_loc, const int32_t *topk_ids,
                    int32_t *counts, int32_t *offsets, int32_t *perm, int32_t *inv_perm)
{
    int64_t S = (int64_t)T * k;
    for (int e = 0; e < E_loc; ++e)
        counts[e] = 0;
    for (int64_t i = 0; i < S; ++i) {
        int e = topk_ids[i] - expert_begin;
        if (e >= 0 && e < E_loc)
            counts[e]++;
    }
    offsets[0] = 0;
    for (int e = 0; e < E_loc; ++e)
        offsets[e + 1] = offsets[e] + counts[e];
    int32_t *cursor = (int32_t *)malloc(sizeof(int32_t) * (size_t)(E_loc > 0 ? E_loc : 1));
    for (int e = 0; e < E_loc; ++e)
        cursor[e] = offsets[e];
    for (int64_t i = 0; i < S; ++i)
        perm[i] = -1;
    for (int t = 0; t < T; ++t) {
        for (int j = 0; j < k; ++j) {
            int64_t slot = (int64_t)t * k + j;
            int e = topk_ids[slot] - expert_begin;
            if (e >= 0 && e < E_loc) {
                int32_t r = cursor[e]++;
                perm[r] = (int32_t)slot;
                inv_perm[slot] = r;
            } else {
                inv_perm[slot] = -1;
            }
        }
    }
    free(cursor);
}

/* ------------------------------------------------------------------ */
/* step 3/4: grouped GEMM over expert slabs                            */
/* ------------------------------------------------------------------ */

enum { ORACLE_W13_SWIGLU = 0, ORACLE_W2 = 1, ORACLE_RAW = 2 };

/*
 * One grouped GEMM. For every local expert e and every row r in
 * [offsets[e], offsets[e+1]) the activation row is a[r] (a_row_index NULL) or
 * a[a_row_index[r] / top_k] (gathered through the permutation), K wide, bf16.
 * Weights of expert e: N rows of K int4 codes with bf16 scales [N][K/G].
 *   kind RAW        : c[r][n] = sum_k a[r][k] W[e][n][k]            (N columns)
 *   kind W2         : same as RAW                                    (N columns)
 *   kind W13_SWIGLU : N = 2I; g = row n, u = row I+n;
 *                     c[r][n] = silu(g) * u                          (I columns)
 * Each result is rounded once from fp64 to c's type: out_f32 != 0 -> binary32,
 * else bf16. Rows whose row_sel entry is 0 are skipped (row_sel may be NULL).
 */
void oracle_grouped_gemm(int kind, int E_loc, int N, int K, int G,
                         const uint16_t *a, const int32_t *a_row_index, int top_k,
                         const int32_t *offsets, const uint8_t *wq, const uint16_t *s,
                         const uint8_t *row_sel, void *c, int out_f32)
{
    int out_cols = (kind == ORACLE_W13_SWIGLU) ? N / 2 : N;
    for (int e = 0; e < E_loc; ++e) {
        int r0 = offsets[e], r1 = offsets[e + 1];
        int any = 0;
        for (int r = r0; r < r1; ++r)
            if (!row_sel || row_sel[r])
                any = 1;
        if (!any)
            continue;
        /* dequantise this expert's slab once (exact) */
        double *W = (double *)malloc(sizeof(double) * (size_t)N * (size_t)K);
#pragma omp parallel for schedule(static)
        for (int n = 0; n < N; ++n)
            for (int kk = 0; kk < K; ++kk)
                W[(int64_t)n * K + kk] = weight(wq, s, N, K, G, e, n, kk);
#pragma omp parallel for schedule(dynamic, 1)
        for (int r = r0; r < r1; ++r) {
            if (row_sel && !row_sel[r])
                continue;
            int64_t src = a_row_index ? (int64_t)(a_row_index[r] / top_k) : (int64_t)r;
            const uint16_t *arow = a + src * K;
            double *x = (double *)malloc(sizeof(double) * (size_t)K);
            for (int kk = 0; kk < K; ++kk)
                x[kk] = bf16_to_double(arow[kk]);
            for (int n = 0; n < out_cols; ++n) {
                double v;
                if (kind == ORACLE_W13_SWIGLU) {
                    double g = 0.0, u = 0.0;
                    const double *wg = W + (int64_t)n * K;
                    const double *wu = W + (int64_t)(n + out_cols) * K;
                    for (int kk = 0; kk < K; ++kk)
                        g += x[kk] * wg[kk];
                    for (int kk = 0; kk < K; ++kk)
                        u += x[kk] * wu[kk];
                    v = silu(g) * u;
                } else {
                    double acc = 0.0;
                    const double *wr = W + (int64_t)n * K;
                    for (int kk = 0; kk < K; ++kk)
                        acc += x[kk] * wr[kk];
                    v = acc;
                }
                if (out_f32)
                    ((float *)c)[(int64_t)r * out_cols + n] = (float)v;
                else
                    ((uint16_t *)c)[(int64_t)r * out_cols + n] = oracle_bf16_from_double(v);
            }
            free(x);
        }
        free(W);
    }
}

/* ------------------------------------------------------------------ */
/* step 5: finalize (weighted unpermute / combine)                     */
/* ------------------------------------------------------------------ */

/*
 * out[t][c] for every token t and column c < H:
 *   the first slot j (in slot order) with inv_perm[t][j] >= 0 gives
 *       acc = y[r][c] * w[t][j]               (binary32 multiply, RNE)
 *   every later present slot gives
 *       acc = fmaf(y[r][c], w[t][j], acc)     (binary32 FMA, one rounding)
 *   then each shared expert s < S (ys[s][t][c], same dtype as y) gives
 *       acc = acc + ys[s][t][c]               (binary32 add = fmaf(v, 1, acc)),
 *       or acc = ys[s][t][c] when it is the first term
 *   no term at all: acc = +0.0.
 * y is bf16 (y_f32 == 0) or binary32; out is binary32 (out_f32 != 0) or the
 * bf16 RNE rounding of acc. No flush-to-zero anywhere. Tokens whose tok_sel
 * entry is 0 are skipped (tok_sel may be NULL).
 */
void oracle_finalize(int T, int k, int H, const void *y, int y_f32, const float *topk_w,
                     const int32_t *inv_perm, int S, const void *ys, const uint8_t *tok_sel, void *out,
                     int out_f32)
{
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        if (tok_sel && !tok_sel[t])
            continue;
        for (int c = 0; c < H; ++c) {
            float acc = 0.0f;
            int first = 1;
            for (int j = 0; j < k; ++j) {
                int32_t r = inv_perm[(int64_t)t * k + j];
                if (r < 0)
                    continue;
                float v = y_f32 ? ((const float *)y)[(int64_t)r * H + c]
                                : (float)bf16_to_double(((const uint16_t *)y)[(int64_t)r * H + c]);
                float w = topk_w[(int64_t)t * k + j];
                if (first) {
                    acc = v * w;
                    first = 0;
                } else {
                    acc = fmaf(v, w, acc);
                }
            }
            for (int sh = 0; sh < S; ++sh) {
                int64_t i = ((int64_t)sh * T + t) * H + c;
                float v = y_f32 ? ((const float *)ys)[i] : (float)bf16_to_double(((const uint16_t *)ys)[i]);
                acc = first ? v : acc + v;
                first = 0;
            }
            if (out_f32)
                ((float *)out)[(int64_t)t * H + c] = acc;
            else
                ((uint16_t *)out)[(int64_t)t * H + c] = oracle_bf16_from_double((double)acc);
        }
    }
}

/* ------------------------------------------------------------------ */
/* the whole layer, through the permutation                            */
/* ------------------------------------------------------------------ */

/*
 * route -> permute -> grouped GEMM (w13 + SwiGLU) -> grouped GEMM (w2) ->
 * finalize. Caller-owned buffers receive every intermediate:
 *   topk_ids, topk_w, inv_perm [T*k]; perm [T*k]; counts [E_loc];
 *   offsets [E_loc+1]; h bf16 [T*k][I]; y bf16 [T*k][H]; out bf16 [T][H].
 * S shared experts (S >= 0; weights w13_sh [S][2I][H/2], s13_sh, w2_sh,
 * s2_sh in the routed layout) run on every token: hs bf16 [S][T][I] and
 * ys bf16 [S][T][H] receive their intermediates (NULL when S == 0).
 * tok_sel (nullable) restricts the expert FFN and the combine to the selected
 * tokens; routing and the permutation always cover every token.
 */
void oracle_layer(int T, int E_g, int k, int expert_begin, int E_loc, int H, int I, int G,
                  const uint16_t *x, const float *logits,
                  const uint8_t *w13_q, const uint16_t *s13, const uint8_t *w2_q, const uint16_t *s2,
                  int S_sh, const uint8_t *w13_sh, const uint16_t *s13_sh, const uint8_t *w2_sh,
                  const uint16_t *s2_sh, const uint8_t *tok_sel,
                  int32_t *topk_ids, float *topk_w, int32_t *counts, int32_t *offsets,
                  int32_t *perm, int32_t *inv_perm, uint16_t *h, uint16_t *y, uint16_t *hs, uint16_t *ys,
                  uint16_t *out)
{
    oracle_route(T, E_g, k, logits, topk_ids, topk_w);
    oracle_permute(T, k, expert_begin, E_loc, topk_ids, counts, offsets, perm, inv_perm);
    int64_t S = (int64_t)T * k;
    uint8_t *row_sel = NULL;
    if (tok_sel) {
        row_sel = (uint8_t *)calloc((size_t)(S > 0 ? S : 1), 1);
        for (int64_t r = 0; r < S; ++r)
            if (perm[r] >= 0 && tok_sel[perm[r] / k])
                row_sel[r] = 1;
    }
    oracle_grouped_gemm(ORACLE_W13_SWIGLU, E_loc, 2 * I, H, G, x, perm, k, offsets, w13_q, s13,
                        row_sel, h, 0);
    oracle_grouped_gemm(ORACLE_W2, E_loc, H, I, G, h, NULL, k, offsets, w2_q, s2, row_sel, y, 0);
    /* each shared expert: one expert holding all T token rows, in token order */
    int32_t one[2] = {0, T};
    for (int sh = 0; sh < S_sh; ++sh) {
        oracle_grouped_gemm(ORACLE_W13_SWIGLU, 1, 2 * I, H, G, x, NULL, 1, one,
                            w13_sh + (int64_t)sh * 2 * I * (H / 2), s13_sh + (int64_t)sh * 2 * I * (H / G),
                            tok_sel, hs + (int64_t)sh * T * I, 0);
        oracle_grouped_gemm(ORACLE_W2, 1, H, I, G, hs + (int64_t)sh * T * I, NULL, 1, one,
                            w2_sh + (int64_t)sh * H * (I / 2), s2_sh + (int64_t)sh * H * (I / G),
                            tok_sel, ys + (int64_t)sh * T * H, 0);
    }
    oracle_finalize(T, k, H, y, 0, topk_w, inv_perm, S_sh, ys, tok_sel, out, 0);
    free(row_sel);
}

/* ------------------------------------------------------------------ */
/* brute force: per token, per slot, no permutation at all             */
/* ------------------------------------------------------------------ */

/*
 * The naive per-(token, expert) MLP: for token t and slot j with a local
 * expert, run that expert's FFN on x[t] directly from the packed weights,
 * then combine the slots in slot order exactly as oracle_finalize does.
 * Routing is taken from topk_ids / topk_w (computed by oracle_route).
 * Same fp64 summation order as the permuted path, so the two must agree
 * bit for bit; any bookkeeping error in the permutation shows up here.
 */
void oracle_layer_bruteforce(int T, int k, int expert_begin, int E_loc, int H, int I, int G,
                             const uint16_t *x, const int32_t *topk_ids, const float *topk_w,
                             const uint8_t *w13_q, const uint16_t *s13,
                             const uint8_t *w2_q, const uint16_t *s2,
                             int S, const uint8_t *w13_sh, const uint16_t *s13_sh,
                             const uint8_t *w2_sh, const uint16_t *s2_sh,
                             const uint8_t *tok_sel, uint16_t *out)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int t = 0; t < T; ++t) {
        if (tok_sel && !tok_sel[t])
            continue;
        double *xv = (double *)malloc(sizeof(double) * (size_t)H);
        double *hv = (double *)malloc(sizeof(double) * (size_t)I);
        float *acc = (float *)calloc((size_t)H, sizeof(float));
        for (int kk = 0; kk < H; ++kk)
            xv[kk] = bf16_to_double(x[(int64_t)t * H + kk]);
        int first = 1;
        for (int j = 0; j < k; ++j) {
            int e = topk_ids[(int64_t)t * k + j] - expert_begin;
            if (e < 0 || e >= E_loc)
                continue;
            for (int n = 0; n < I; ++n) {
                double g = 0.0, u = 0.0;
                for (int kk = 0; kk < H; ++kk)
                    g += xv[kk] * weight(w13_q, s13, 2 * I, H, G, e, n, kk);
                for (int kk = 0; kk < H; ++kk)
                    u += xv[kk] * weight(w13_q, s13, 2 * I, H, G, e, I + n, kk);
                hv[n] = bf16_to_double(oracle_bf16_from_double(silu(g) * u));
            }
            float w = topk_w[(int64_t)t * k + j];
            for (int c = 0; c < H; ++c) {
                double d = 0.0;
                for (int n = 0; n < I; ++n)
                    d += hv[n] * weight(w2_q, s2, H, I, G, e, c, n);
                float v = (float)bf16_to_double(oracle_bf16_from_double(d));
                acc[c] = first ? v * w : fmaf(v, w, acc[c]);
            }
            first = 0;
        }
        /* shared experts: the same FFN on every token, weight 1, after the slots */
        for (int sh = 0; sh < S; ++sh) {
            for (int n = 0; n < I; ++n) {
                double g = 0.0, u = 0.0;
                for (int kk = 0; kk < H; ++kk)
                    g += xv[kk] * weight(w13_sh, s13_sh, 2 * I, H, G, sh, n, kk);
                for (int kk = 0; kk < H; ++kk)
                    u += xv[kk] * weight(w13_sh, s13_sh, 2 * I, H, G, sh, I + n, kk);
                hv[n] = bf16_to_double(oracle_bf16_from_double(silu(g) * u));
            }
            for (int c = 0; c < H; ++c) {
                double d = 0.0;
                for (int n = 0; n < I; ++n)
                    d += hv[n] * weight(w2_sh, s2_sh, H, I, G, sh, c, n);
                float v = (float)bf16_to_double(oracle_bf16_from_double(d));
                acc[c] = first ? v : acc[c] + v;
            }
            first = 0;
        }
        for (int c = 0; c < H; ++c)
            out[(int64_t)t * H + c] = oracle_bf16_from_double((double)acc[c]);
        free(acc);
        free(hv);
        free(xv);
    }
}

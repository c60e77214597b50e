/*
 * mxfp4_oracle.c -- plain CPU oracle for the W4A4 (MXFP4) variant of the
 * Mixture-of-Experts expert layer.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library. The GPU product path
 * never calls it and shares no code, header, table or helper with it.
 *
 * Pages followed (cited by title and section):
 *   [FI]  "FlashInfer, CuTe DSL W4A16 MoE optimization and bitwise-exactness
 *         tests" (FlashInfer PR #7196 analysis): section 2 ("Arithmetic
 *         Alignment": W4A4 and W4A16 finalizers share the combine) and the
 *         performance section (a TRTLLM W4A4 kernel beside the W4A16 one).
 *   [GC]  "GC-MoE: ... FP8/FP4 Grouped GEMM via CUDA Green Contexts"
 *         (abstract): FP4 block-scaled matrix multiplies, 4-bit operands
 *         decoded in registers, activations requantized between the GEMMs.
 * The pages fix no FP4 encoding. Reading taken (also in the design notes):
 * the OCP Microscaling (MX) format MXFP4 --
 *   element  E2M1: sign bit, 2 exponent bits (bias 1), 1 mantissa bit; a
 *            zero exponent field is subnormal (value = mantissa/2), so the
 *            magnitudes are 0, 0.5, 1, 1.5, 2, 3, 4, 6;
 *   scale    E8M0: one unsigned byte s per block, value 2^(s - 127) (s = 255,
 *            NaN, is never produced here);
 *   block    32 consecutive elements along K;
 *   quantizing a block V_0..V_31: X = 2^(floor(log2(max |V_i|)) - 2) (2 is
 *            the largest E2M1 exponent), the exponent clamped to [-127, 127];
 *            each V_i / X rounded to the nearest E2M1 magnitude, ties to the
 *            even code, magnitudes past 6 kept at 6 (saturation), the sign
 *            of V_i kept; an all-zero block takes s = 0.
 * Weights: codes in the int4 byte layout (element k in byte k/2, even k in
 * the low nibble) holding E2M1 codes; scales uint8 [E][N][K/32].
 * The W4A4 layer: each token's bf16 activation row is quantized (per 32 along
 * H); the gate/up GEMM gives h = bf16(silu(g) * u) exactly as in the W4A16
 * layer; h is requantized per 32 along I; the down GEMM gives y in bf16; the
 * combine is the W4A16 layer's (fp32 multiply, then FMA, slot order).
 *
 * Arithmetic: dequantised operands and their products are exact in fp64;
 * every dot product is an fp64 sum in ascending k (exact for the operand and
 * scale ranges drawn here), then one rounding to the stored type.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* from moe_oracle.c (same library) */
uint16_t oracle_bf16_from_double(double d);
void oracle_route(int T, int E, int k, const float *logits, int32_t *topk_ids, float *topk_w);
void oracle_permute(int T, int k, int expert_begin, int E_loc, const int32_t *topk_ids, int32_t *counts,
                    int32_t *offsets, int32_t *perm, int32_t *inv_perm);
void oracle_finalize(int T, int k, int H, const void *y, int y_f32, const float *topk_w, const int32_t *inv_perm,
                     int S, const void *ys, const uint8_t *tok_sel, void *out, int out_f32);

static double bf16_value(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* E2M1 code (4 bits) -> value, from its sign / exponent / mantissa fields. */
double oracle_e2m1_value(int code)
{
    const int sign = (code >> 3) & 1, ex = (code >> 1) & 3, man = code & 1;
    const double mag = ex == 0 ? 0.5 * man : ldexp(1.0 + 0.5 * man, ex - 1);
    return sign ? -mag : mag;
}

/* E8M0 scale byte -> 2^(s - 127). */
double oracle_e8m0_value(int s) { return ldexp(1.0, s - 127); }

/* Element k of a row of E2M1 codes (two per byte, even k in the low nibble). */
static int code_at(const uint8_t *row, int64_t k)
{
    const uint8_t b = row[k / 2];
    return (k & 1) ? (b >> 4) : (b & 0x0F);
}

/*
 * Quantize `rows` rows of K bf16 values (K a multiple of 32) to MXFP4: codes
 * [rows][K/2], scales [rows][K/32]. Each element is rounded by searching
 * the eight magnitudes for the nearest one (a tie goes to the even code).
 */
void oracle_mx_quantize(int64_t rows, int K, const uint16_t *x, uint8_t *codes, uint8_t *scales)
{
    const int nb = K / 32;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const uint16_t *xr = x + r * K;
        uint8_t *cr = codes + r * (K / 2);
        memset(cr, 0, (size_t)(K / 2));
        for (int b = 0; b < nb; ++b) {
            double amax = 0.0;
            for (int i = 0; i < 32; ++i) {
                const double a = fabs(bf16_value(xr[b * 32 + i]));
                if (a > amax)
                    amax = a;
            }
            int ex = -127;
            if (amax > 0.0) {
                int e2;
                (void)frexp(amax, &e2);           /* amax = m 2^e2, m in [0.5, 1): floor(log2) = e2 - 1 */
                ex = (e2 - 1) - 2;
                if (ex < -127)
                    ex = -127;
                if (ex > 127)
                    ex = 127;
            }
            scales[r * nb + b] = (uint8_t)(ex + 127);
            for (int i = 0; i < 32; ++i) {
                const double v = bf16_value(xr[b * 32 + i]);
                const double p = fabs(v) / ldexp(1.0, ex);
                int best = 0;
                double bestd = INFINITY;
                for (int c = 0; c < 8; ++c) {         /* nearest magnitude; equal distance: keep the even code */
                    const double d = fabs(p - oracle_e2m1_value(c));
                    if (d < bestd || (d == bestd && (c & 1) == 0 && (best & 1) != 0)) {
                        best = c;
                        bestd = d;
                    }
                }
                if (p > 6.0)
                    best = 7;                         /* saturation */
                const int code = best | (signbit(v) ? 8 : 0);
                const int k = b * 32 + i;
                cr[k / 2] |= (uint8_t)(code << ((k & 1) ? 4 : 0));
            }
        }
    }
}

/* Dequantised MXFP4 element k of a row: code value * 2^(scale - 127). */
static double mx_value(const uint8_t *codes_row, const uint8_t *scales_row, int64_t k)
{
    return oracle_e2m1_value(code_at(codes_row, k)) * oracle_e8m0_value(scales_row[k / 32]);
}

static double silu(double z) { return z / (1.0 + exp(-z)); }

enum { MX_W13_SWIGLU = 0, MX_W2 = 1, MX_RAW = 2 };

/*
 * Grouped GEMM on MXFP4 operands. For local expert e and rows r in
 * [offsets[e], offsets[e+1]) the activation row is row a_row_index[r] / top_k
 * of (a_codes, a_scales) (or row r when a_row_index is NULL). Weights of
 * expert e: N rows of K E2M1 codes (wq [E][N][K/2]) with scales ws [E][N][K/32].
 *   RAW / W2   : c[r][n] = sum_k A[r][k] W[e][n][k]       (N columns)
 *   W13_SWIGLU : N = 2I, c[r][n] = silu(g_n) * u_n with g row n, u row I + n
 * One rounding from fp64 to c's type (binary32 or bf16). Rows with row_sel 0
 * are skipped (row_sel may be NULL).
 */
void oracle_grouped_gemm_mxfp4(int kind, int E_loc, int N, int K, const uint8_t *a_codes, const uint8_t *a_scales,
                               const int32_t *a_row_index, int top_k, const int32_t *offsets, const uint8_t *wq,
                               const uint8_t *ws, const uint8_t *row_sel, void *c, int out_f32)
{
    const int out_cols = kind == MX_W13_SWIGLU ? N / 2 : N;
    for (int e = 0; e < E_loc; ++e) {
#pragma omp parallel for schedule(dynamic, 1)
        for (int r = offsets[e]; r < offsets[e + 1]; ++r) {
            if (row_sel && !row_sel[r])
                continue;
            const int64_t src = a_row_index ? (int64_t)(a_row_index[r] / top_k) : (int64_t)r;
            double *x = (double *)malloc(sizeof(double) * (size_t)K);
            for (int64_t k = 0; k < K; ++k)
                x[k] = mx_value(a_codes + src * (K / 2), a_scales + src * (K / 32), k);
            for (int n = 0; n < out_cols; ++n) {
                double v;
                if (kind == MX_W13_SWIGLU) {
                    double g = 0.0, u = 0.0;
                    const int64_t rg = (int64_t)e * N + n, ru = (int64_t)e * N + n + out_cols;
                    for (int64_t k = 0; k < K; ++k)
                        g += x[k] * mx_value(wq + rg * (K / 2), ws + rg * (K / 32), k);
                    for (int64_t k = 0; k < K; ++k)
                        u += x[k] * mx_value(wq + ru * (K / 2), ws + ru * (K / 32), k);
                    v = silu(g) * u;
                } else {
                    double acc = 0.0;
                    const int64_t rw = (int64_t)e * N + n;
                    for (int64_t k = 0; k < K; ++k)
                        acc += x[k] * mx_value(wq + rw * (K / 2), ws + rw * (K / 32), k);
                    v = acc;
                }
                if (out_f32)
                    ((float *)c)[(int64_t)r * out_cols + n] = (float)v;
                else
                    ((uint16_t *)c)[(int64_t)r * out_cols + n] = oracle_bf16_from_double(v);
            }
            free(x);
        }
    }
}

/*
 * The W4A4 layer through the permutation: route -> permute -> quantize x ->
 * gate/up GEMM (+ SwiGLU, h bf16) -> requantize h -> down GEMM (y bf16) ->
 * finalize. Buffers receive every intermediate: topk_ids, topk_w, inv_perm
 * [T*k]; counts [E_loc]; offsets [E_loc+1]; perm [T*k]; xq [T][H/2], xs
 * [T][H/32]; h bf16 [T*k][I]; hq [T*k][I/2], hsc [T*k][I/32]; y bf16
 * [T*k][H]; out bf16 [T][H]. tok_sel (nullable) restricts the expert FFN and
 * the combine to the selected tokens.
 */
void oracle_layer_w4a4(int T, int E_g, int k, int expert_begin, int E_loc, int H, int I, const uint16_t *x,
                       const float *logits, const uint8_t *w13_q, const uint8_t *w13_s, const uint8_t *w2_q,
                       const uint8_t *w2_s, const uint8_t *tok_sel, int32_t *topk_ids, float *topk_w,
                       int32_t *counts, int32_t *offsets, int32_t *perm, int32_t *inv_perm, uint8_t *xq,
                       uint8_t *xs, uint16_t *h, uint8_t *hq, uint8_t *hsc, uint16_t *y, uint16_t *out)
{
    oracle_route(T, E_g, k, logits, topk_ids, topk_w);
    oracle_permute(T, k, expert_begin, E_loc, topk_ids, counts, offsets, perm, inv_perm);
    const int64_t S = (int64_t)T * k;
    uint8_t *row_sel = NULL;
    if (tok_sel) {
        row_sel = (uint8_t *)calloc((size_t)(S > 0 ? S : 1), 1);
        for (int64_t r = 0; r < S; ++r)
            if (perm[r] >= 0 && tok_sel[perm[r] / k])
                row_sel[r] = 1;
    }
    oracle_mx_quantize(T, H, x, xq, xs);
    oracle_grouped_gemm_mxfp4(MX_W13_SWIGLU, E_loc, 2 * I, H, xq, xs, perm, k, offsets, w13_q, w13_s, row_sel, h, 0);
    oracle_mx_quantize(S, I, h, hq, hsc);
    oracle_grouped_gemm_mxfp4(MX_W2, E_loc, H, I, hq, hsc, NULL, k, offsets, w2_q, w2_s, row_sel, y, 0);
    oracle_finalize(T, k, H, y, 0, topk_w, inv_perm, 0, NULL, tok_sel, out, 0);
    free(row_sel);
}

/*
 * The same layer per token and slot, with no permutation: quantize x[t],
 * run the slot's expert on it (h row bf16, requantized, y row bf16), combine
 * the slots in slot order as the finalize does. Must equal
 * oracle_layer_w4a4 bit for bit (same fp64 sums in the same order).
 */
void oracle_layer_w4a4_bruteforce(int T, int k, int expert_begin, int E_loc, int H, int I, const uint16_t *x,
                                  const int32_t *topk_ids, const float *topk_w, const uint8_t *w13_q,
                                  const uint8_t *w13_s, const uint8_t *w2_q, const uint8_t *w2_s,
                                  const uint8_t *tok_sel, uint16_t *out)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int t = 0; t < T; ++t) {
        if (tok_sel && !tok_sel[t])
            continue;
        uint8_t *xq = (uint8_t *)malloc((size_t)H / 2), *xs = (uint8_t *)malloc((size_t)H / 32);
        uint8_t *hq = (uint8_t *)malloc((size_t)I / 2), *hsc = (uint8_t *)malloc((size_t)I / 32);
        uint16_t *hrow = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)I);
        float *acc = (float *)calloc((size_t)H, sizeof(float));
        oracle_mx_quantize(1, H, x + (int64_t)t * H, xq, xs);
        int first = 1;
        for (int j = 0; j < k; ++j) {
            const int e = topk_ids[(int64_t)t * k + j] - expert_begin;
            if (e < 0 || e >= E_loc)
                continue;
            for (int n = 0; n < I; ++n) {
                double g = 0.0, u = 0.0;
                const int64_t rg = (int64_t)e * 2 * I + n, ru = rg + I;
                for (int64_t kk = 0; kk < H; ++kk) {
                    const double a = mx_value(xq, xs, kk);
                    g += a * mx_value(w13_q + rg * (H / 2), w13_s + rg * (H / 32), kk);
                }
                for (int64_t kk = 0; kk < H; ++kk) {
                    const double a = mx_value(xq, xs, kk);
                    u += a * mx_value(w13_q + ru * (H / 2), w13_s + ru * (H / 32), kk);
                }
                hrow[n] = oracle_bf16_from_double(silu(g) * u);
            }
            oracle_mx_quantize(1, I, hrow, hq, hsc);
            const float w = topk_w[(int64_t)t * k + j];
            for (int c = 0; c < H; ++c) {
                double d = 0.0;
                const int64_t rw = (int64_t)e * H + c;
                for (int64_t n = 0; n < I; ++n)
                    d += mx_value(hq, hsc, n) * mx_value(w2_q + rw * (I / 2), w2_s + rw * (I / 32), n);
                const float v = (float)bf16_value(oracle_bf16_from_double(d));
                acc[c] = first ? v * w : fmaf(v, w, acc[c]);
            }
            first = 0;
        }
        for (int c = 0; c < H; ++c)
            out[(int64_t)t * H + c] = oracle_bf16_from_double((double)acc[c]);
        free(acc);
        free(hrow);
        free(hsc);
        free(hq);
        free(xs);
        free(xq);
    }
}

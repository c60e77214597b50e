/*
 * moe_w4a16.h -- C ABI of the MI355X (gfx950) W4A16 Mixture-of-Experts
 * expert layer: top-k routing, stable expert permutation, grouped GEMM over
 * expert slabs on int4 group-scaled weights with bf16 activations (gate/up
 * with fused SwiGLU, then down), and the slot-ordered finalize combine.
 *
 * Pages that define the operations (cited by title and section):
 *   [FI] "FlashInfer, CuTe DSL W4A16 MoE optimization and bitwise-exactness
 *        tests" (FlashInfer PR #7196 analysis): section 1 `moe_finalize.py`
 *        (combine: fp32 multiply for the first slot, fp32 FMA for later slots
 *        in slot order, no flush-to-zero); section 2 `moe_w4a16_kernel.py`
 *        (runtime MMA N from the routed-token count, skipping inactive
 *        subtiles; valid-rows-only bf16 permutation; SwiGLU); section 3
 *        (zero-tolerance checks).
 *   [IL] "T2-1-3 Qwen3-MoE inference optimization report" (InfiniLM PR #500):
 *        section 2.2 (bucket the routing ids into per-expert counts and a
 *        permutation, gather, grouped GEMMs gate/up/down + SwiGLU, weighted
 *        scatter back to tokens; grouped_gemm takes group sizes); section
 *        2.3 (the host-side count passthrough that skips a device-to-host
 *        sync -- here counts never leave the device at all).
 *   [GC] "GC-MoE: Overlapping Expert-Parallel Token Dispatch with FP8/FP4
 *        Grouped GEMM via CUDA Green Contexts" (abstract): decode holds 1-256
 *        tokens per rank and is dominated by weight traffic; operand-swapped
 *        MMA; in-register 4-bit decode fed to the matrix unit; fused SwiGLU.
 *   [FI2] "FlashInfer, NVFP4 SVDQuant GEMM kernel optimization: per-
 *        architecture dispatch" (FlashInfer PR #6986 analysis), section 1:
 *        `is_supported` answers a shape query without raising; `run` raises.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are caller-owned DEVICE memory, 16-byte aligned
 *     (workspace: 256-byte aligned). The library never allocates, frees or
 *     synchronises and never reads device data on the host.
 *   - All work is enqueued on `stream` (a hipStream_t; NULL = the null
 *     stream) and the call returns after launching, so the calls can be
 *     captured into a HIP graph. No memset nodes are issued.
 *   - Host-side validation failures return an error BEFORE any launch, so
 *     outputs are untouched. A launch failure returns MOE_ERR_HIP. Faults
 *     inside kernels surface at the caller's next synchronisation.
 *   - The library is stateless; calls are thread-safe.
 *
 * Storage formats (row-major, contiguous):
 *   bf16 values are 16-bit patterns (uint16_t here).
 *   int4 weights: two's-complement codes in [-8, 7], element k of a row in
 *   byte k/2, even k in the low nibble, K contiguous; no zero point.
 *   Scales: one bf16 per (weight row, 128-wide K group): W[n][k] =
 *   q[n][k] * s[n][k/128].
 *   w13_q  uint8 [E_loc][2*I][H/2], s13 bf16 [E_loc][2*I][H/128]: rows
 *          [0, I) are the gate projection, [I, 2I) the up projection.
 *   w2_q   uint8 [E_loc][H][I/2],   s2  bf16 [E_loc][H][I/128].
 *   Weight arrays start at local expert 0 (global id expert_begin).
 *
 * Tiled code layout (moe_shape.weight_layout == MOE_WEIGHTS_TILED; scales
 * keep the plain layout above). The codes of a weight matrix with N rows and
 * K columns, reordered so that one 64-lane load of 16 bytes per lane reads
 * 1 KiB contiguously, and so that each 32-bit word holds its 8 codes in the
 * order the matrix unit consumes them:
 *   run(e, b, g, i, l) = plain[e][row(16*(8*b+i), l%16)][64*g + 16*(l/16) .. +16)
 *   tiled[e][b][g][i][l][4*w .. 4*w+4) = shuffle(word w of run(e, b, g, i, l)), w < 4
 *   b < N/128 (blocks of 8 sixteen-row tiles), g < K/128, i < 8, l < 64,
 *   row(t0, n) = t0 + n                           for MOE_GEMM_W2 / W13_RAW,
 *   row(16*t, n) = 8*t + n (n < 8), I + 8*t + n - 8 (n >= 8)
 *                                                 for MOE_GEMM_W13_SWIGLU
 *   (a gate row and its up row share a tile). A plain little-endian word
 *   holds codes c0..c7 of 8 consecutive columns, c_j in bits [4j, 4j+4);
 *   shuffle() puts the even codes c0, c2, c4, c6 in nibbles 0..3 and the odd
 *   codes c1, c3, c5, c7 in nibbles 4..7, so that nibble pairs (j, j+4) are
 *   column pairs (2j, 2j+1). moe_w4a16_pack_weights writes it; it is an
 *   offline, once-per-model step.
 */
#ifndef MOE_W4A16_H
#define MOE_W4A16_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_NULL = 1,        /* a required pointer is NULL                     */
    MOE_ERR_SHAPE = 2,       /* sizes inconsistent or out of range             */
    MOE_ERR_UNSUPPORTED = 3, /* valid but not supported (group != 128, ...)    */
    MOE_ERR_ALIGN = 4,       /* a pointer violates its alignment requirement   */
    MOE_ERR_WORKSPACE = 5,   /* workspace too small                            */
    MOE_ERR_HIP = 6          /* a kernel launch failed                         */
} moe_status;

typedef enum { MOE_BF16 = 0, MOE_F32 = 1 } moe_dtype;

typedef enum {
    MOE_GEMM_W13_SWIGLU = 0, /* a[R][H] x w13^T -> h[R][I] = bf16(silu(g) * u)  */
    MOE_GEMM_W2 = 1,         /* a[R][I] x w2^T  -> c[R][H] (bf16 or f32)         */
    MOE_GEMM_W13_RAW = 2     /* a[R][H] x w13^T -> c[R][2I] (no activation)      */
} moe_gemm_kind;

typedef enum {
    MOE_WEIGHTS_PLAIN = 0,     /* row-major codes (the storage format above)     */
    MOE_WEIGHTS_TILED = 1      /* codes reordered by moe_w4a16_pack_weights      */
} moe_weight_layout;

typedef struct {
    int32_t num_tokens;        /* T >= 0                                         */
    int32_t hidden;            /* H, multiple of 128, <= 16384                   */
    int32_t inter;             /* I, multiple of 128, <= 16384                   */
    int32_t num_experts;       /* E_g: router logit columns, 1..1024             */
    int32_t expert_begin;      /* global id of local expert 0                    */
    int32_t num_local_experts; /* E_loc, 1..1024, expert_begin+E_loc <= E_g      */
    int32_t top_k;             /* 1..min(E_g, 16)                                */
    int32_t group_size;        /* quantisation group along K: 128 only           */
    int32_t weight_layout;     /* moe_weight_layout of w13_q / w2_q / wq         */
} moe_shape;

/* Human-readable name of a status code (static string, never NULL). The
 * status split follows [FI2] section 1: a run entry point reports a failure
 * (here as a code, which the Python binding raises), while is_supported
 * answers without failing. Unknown codes give "unknown moe_status". */
const char *moe_status_str(moe_status s);

/* Validate a shape without raising: MOE_OK if every entry point supports it,
 * else the status forward() would return ([FI2] section 1: is_supported). */
moe_status moe_w4a16_check_shape(const moe_shape *shape);

/* 1 if moe_w4a16_check_shape(shape) == MOE_OK, else 0. Never an error. */
int moe_w4a16_is_supported(const moe_shape *shape);

/* Bytes of workspace moe_w4a16_forward needs for this shape (0 if the shape
 * is invalid). It holds the layer's intermediates that [IL] section 2.2
 * names between its steps: the routing ids and weights, the per-expert counts
 * and offsets, the permutation and its inverse, the SwiGLU output h [T*k][I]
 * and the expert outputs y [T*k][H] (bf16), plus the permutation's per-range
 * counts for many tokens. Layout is private to the library; the caller owns
 * the memory, and the workspace holds no state from one call to the next. */
size_t moe_w4a16_workspace_size(const moe_shape *shape);

/*
 * The whole layer ([IL] section 2.2: route, bucket by expert, gate/up grouped
 * GEMM with SwiGLU, down grouped GEMM, weighted combine back to tokens; [FI]
 * section 1: the combine's slot order; [GC] abstract: the 1-256 token decode
 * regime it is tuned for): route -> permute -> GEMM1 (w13, SwiGLU) -> GEMM2
 * (w2) -> finalize, all on `stream`, no host synchronisation.
 *   x             bf16  [T][H]        activations
 *   router_logits f32   [T][E_g]
 *   w13_q, s13, w2_q, s2              local experts' weights (formats above;
 *                                     codes plain or tiled per weight_layout)
 *   out           bf16  [T][H]        written for every token; a token with no
 *                                     local slot gets +0.0
 *   workspace     >= moe_w4a16_workspace_size(shape) bytes, 256-B aligned
 * T == 0 is a no-op returning MOE_OK.
 */
moe_status moe_w4a16_forward(const moe_shape *shape, const uint16_t *x, const float *router_logits,
                             const uint8_t *w13_q, const uint16_t *s13, const uint8_t *w2_q,
                             const uint16_t *s2, uint16_t *out, void *workspace,
                             size_t workspace_bytes, void *stream);

/*
 * The layer for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same computation and result as moe_w4a16_forward, with the workspace taken
 * from a fixed device array inside the library, MOE_NOALLOC_SCRATCH_BYTES
 * per GPU (each GPU the library runs on holds one until the process ends).
 * It allocates nothing. A shape whose moe_w4a16_workspace_size exceeds the
 * array returns MOE_ERR_WORKSPACE before any launch (for the Qwen3-30B-A3B
 * expert shape, up to 1484 tokens). Every call on one GPU shares that GPU's
 * array, so calls that overlap on one GPU (two streams, two host threads)
 * race: the caller must order them. The array keeps the last call's
 * intermediates; nothing in it has to start at zero.
 */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
moe_status moe_w4a16_forward_noalloc(const moe_shape *shape, const uint16_t *x, const float *router_logits,
                                     const uint8_t *w13_q, const uint16_t *s13, const uint8_t *w2_q,
                                     const uint16_t *s2, uint16_t *out, void *stream);

/*
 * The layer with shared experts ([GC] abstract: optional, fused shared
 * experts; the reading taken): num_shared (1..4) always-on experts with the
 * routed experts' shape and formats run on every token, and each one's bf16
 * output is added to the binary32 combine with weight 1 after the routed
 * slots (acc = acc + v, or v for a token's first term). They run inside the
 * same launches as the routed experts (extra experts of the grouped GEMMs).
 *   w13_sh [num_shared][2*I][H/2], s13_sh [num_shared][2*I][H/128],
 *   w2_sh  [num_shared][H][I/2],   s2_sh  [num_shared][H][I/128]
 *   (codes plain or tiled per weight_layout, like the routed weights)
 *   workspace >= moe_w4a16_workspace_size_shared(shape, num_shared) bytes
 * Everything else as moe_w4a16_forward. Under expert parallelism pass the
 * shared experts only on the rank that owns the tokens.
 */
size_t moe_w4a16_workspace_size_shared(const moe_shape *shape, int32_t num_shared);
moe_status moe_w4a16_forward_shared(const moe_shape *shape, int32_t num_shared, const uint16_t *x,
                                    const float *router_logits, const uint8_t *w13_q, const uint16_t *s13,
                                    const uint8_t *w2_q, const uint16_t *s2, const uint8_t *w13_sh,
                                    const uint16_t *s13_sh, const uint8_t *w2_sh, const uint16_t *s2_sh,
                                    uint16_t *out, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Top-k routing ([FI] section 2; the layer definition: softmax over all E_g
 * experts, keep the top-k, renormalise). Selection order: larger logit first,
 * lower expert index first among equal logits (-0 == +0); the i-th selected
 * expert is slot i. topk_w[t][i] = exp(l_i - l_0) / sum_{j<k} exp(l_j - l_0)
 * in fp32 (equal to the renormalised softmax up to rounding).
 *   logits f32 [T][E_g] -> topk_ids int32 [T][k] (global ids), topk_w f32 [T][k]
 */
moe_status moe_route(const moe_shape *shape, const float *logits, int32_t *topk_ids,
                     float *topk_w, void *stream);

/*
 * Workspace bytes moe_permute needs: 0 for a shape it permutes in one
 * workgroup, else int32 counts per (token range, local expert) for the
 * parallel path over many tokens (at most 64 ranges, so at most
 * 256 * E_loc bytes). 0 if the shape is invalid. The workspace holds no state
 * between calls; calls that share one on a stream run in order.
 */
size_t moe_permute_workspace_size(const moe_shape *shape);

/*
 * Stable expert permutation ([IL] section 2.2; [FI] section 2 permutation).
 * Slots (t, j) routed to local experts [expert_begin, expert_begin+E_loc) are
 * bucketed by expert, token-ascending within each expert.
 *   topk_ids int32 [T][k] ->
 *   counts   int32 [E_loc]      slots per local expert
 *   offsets  int32 [E_loc+1]    exclusive scan of counts; R = offsets[E_loc]
 *   perm     int32 [T*k]        row r < R holds slot id t*k+j; rows >= R get -1
 *   inv_perm int32 [T][k]       row of slot (t, j), or -1 if not local
 *   x / x_perm (both NULL, or both set): x bf16 [T][H] gathered into
 *                x_perm bf16 [T*k][H], row r = x[perm[r] / k] (rows >= R
 *                untouched)
 * Bit-exact and deterministic (no atomics decide a position).
 * workspace: device memory of moe_permute_workspace_size(shape) bytes,
 * 4-byte aligned (NULL if that is 0); smaller -> MOE_ERR_WORKSPACE.
 */
moe_status moe_permute(const moe_shape *shape, const int32_t *topk_ids, const uint16_t *x,
                       int32_t *counts, int32_t *offsets, int32_t *perm, int32_t *inv_perm,
                       uint16_t *x_perm, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Grouped GEMM over expert slabs with int4 group-scaled weights and bf16
 * activations ([IL] section 2.2 grouped_gemm with group sizes; [FI] section
 * 2 runtime N; [GC] abstract: in-register 4-bit decode fed to the matrix
 * unit). For local expert e and rows r in [offsets[e], offsets[e+1]):
 *   A row r = a[a_row_index[r] / top_k]   if a_row_index != NULL (gather
 *             straight from the unpermuted activations through perm)
 *           = a[r]                         otherwise.
 *   W13_SWIGLU: K = H, weights w13 (2I rows); c = h bf16 [T*k][I] with
 *               h = bf16(silu(g) * u), g = A.W_gate^T, u = A.W_up^T.
 *   W13_RAW:    K = H, c [T*k][2I] = A.w13^T, bf16 or f32 (c_dtype).
 *   W2:         K = I, c [T*k][H]  = A.w2^T,  bf16 or f32 (c_dtype).
 * Accumulation is fp32 over exact int4 codes; the scale of each 128-wide
 * group is applied in fp32. Rows >= R of c are untouched. `offsets` stays on
 * the device: the grid never depends on the counts. The call takes no
 * workspace: every kernel keeps its work list and partial sums in LDS and
 * registers (each workgroup derives its items from `offsets`).
 */
moe_status moe_grouped_gemm_w4a16(const moe_shape *shape, moe_gemm_kind kind, const uint16_t *a,
                                  const int32_t *a_row_index, const int32_t *offsets,
                                  const uint8_t *wq, const uint16_t *s, void *c, moe_dtype c_dtype,
                                  void *stream);

/*
 * Dense W4A16 GEMM: one weight matrix, every row of `a` through it, no
 * routing ([FI] sections 2-3: the MoE GEMM and the dense GEMM share one
 * W4A16 reference; here the dense case runs the grouped kernels with one
 * expert holding all M rows).
 *   c[m][n] = sum_k a[m][k] * W[n][k],  W[n][k] = q[n][k] * s[n][k/128]
 *   M >= 0 (0: no-op); N, K multiples of 128, <= 65536; N*K/2 and M*K*2
 *   below 2^31 bytes (MOE_ERR_UNSUPPORTED beyond)
 *   a   bf16 [M][K]
 *   wq  uint8 [N][K/2], the int4 format above (plain), or tiled by
 *       moe_w4a16_pack_weights with kind MOE_GEMM_W2 and a shape with
 *       E_loc = 1, hidden = N, inter = K (weight_layout says which)
 *   s   bf16 [N][K/128]
 *   c   [M][N], bf16 (RNE) or f32 (c_dtype)
 * Accumulation as in moe_grouped_gemm_w4a16 (exact int4 codes, fp32 sums,
 * the group scale applied in fp32).
 */
moe_status moe_w4a16_dense_gemm(int32_t M, int32_t N, int32_t K, const uint16_t *a, const uint8_t *wq,
                                const uint16_t *s, void *c, moe_dtype c_dtype, int32_t weight_layout,
                                void *stream);

/*
 * Finalize: weighted unpermute / combine ([FI] section 1 `moe_finalize.py`).
 * For every token t and column c < H: the first slot j (slot order) with
 * inv_perm[t][j] >= 0 gives acc = y[r][c] * w[t][j] (IEEE binary32 multiply,
 * round to nearest even); each later present slot gives
 * acc = fma(y[r][c], w[t][j], acc) (IEEE binary32 FMA); no slot -> +0.0.
 * No flush-to-zero: subnormal inputs, products and sums are kept.
 *   y       [T*k][H]  bf16 or f32 (y_dtype); the whole array must be
 *                     readable (the kernel may read row 0 for an absent slot
 *                     and discard it)
 *   topk_w  f32 [T][k], inv_perm int32 [T][k]
 *   out     [T][H]    f32 (the accumulator) or bf16 (its RNE rounding)
 * Bit-exact against the IEEE definition.
 */
moe_status moe_finalize(const moe_shape *shape, const void *y, moe_dtype y_dtype,
                        const float *topk_w, const int32_t *inv_perm, void *out,
                        moe_dtype out_dtype, void *stream);

/*
 * Reorder one weight matrix's int4 codes from the plain layout into the tiled
 * layout described above (an internal layout of the grouped GEMM, like the
 * kernel layout [FI] section 3 inverts back to a plain one in its tests).
 *   kind    MOE_GEMM_W13_SWIGLU (w13, gate/up rows paired in tiles),
 *           MOE_GEMM_W13_RAW (w13, rows in order) or MOE_GEMM_W2 (w2)
 *   wq      uint8 plain codes of the shape's E_loc experts
 *   wq_tiled uint8, same size, must not overlap wq
 * shape->weight_layout is ignored. The GEMM and the layer then take
 * wq_tiled with weight_layout = MOE_WEIGHTS_TILED (w13 packed with
 * MOE_GEMM_W13_SWIGLU for the layer and for W13_SWIGLU GEMMs, with
 * MOE_GEMM_W13_RAW for W13_RAW GEMMs). Bit-exact byte permutation.
 */
moe_status moe_w4a16_pack_weights(const moe_shape *shape, moe_gemm_kind kind, const uint8_t *wq,
                                  uint8_t *wq_tiled, void *stream);

/*
 * ---- The W4A4 variant: MXFP4 weights and activations ----------------------
 * [FI] section 2 ("Arithmetic Alignment": W4A4 finalizers beside the W4A16
 * ones) and its performance section (a W4A4 kernel); [GC] abstract (FP4
 * block-scaled grouped GEMMs, activations requantized between the GEMMs).
 * The pages fix no FP4 encoding; the format read is the OCP MX one, MXFP4:
 *   element  E2M1 (sign, 2 exponent bits with bias 1, 1 mantissa bit; a zero
 *            exponent field is subnormal): magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6;
 *            codes two per byte, element k of a row in byte k/2, even k in the
 *            low nibble (the int4 byte layout), rows K-contiguous;
 *   scale    E8M0 byte s per 32 consecutive elements along K: 2^(s - 127);
 *   weights  w13_q uint8 [E_loc][2*I][H/2], w13_s uint8 [E_loc][2*I][H/32],
 *            w2_q  uint8 [E_loc][H][I/2],   w2_s  uint8 [E_loc][H][I/32].
 * These entry points take moe_shape.group_size == 32 (else
 * MOE_ERR_UNSUPPORTED); H and I stay multiples of 128. weight_layout ==
 * MOE_WEIGHTS_TILED selects the tiled MXFP4 code layout (scales stay plain):
 * the int4 tiled layout's runs without the word shuffle (a lane's 16 bytes
 * are its operand of the scaled matrix instruction as they lie),
 *   tiled[e][b][g][i][l][0 .. 16) = plain[e][row(16*(8*b+i), l%16)][64*g + 16*(l/16) .. +16)
 * with b, g, i, l and row() as above; moe_mxfp4_pack_weights writes it.
 */

/*
 * Quantize rows x rows of K bf16 values (K a multiple of 32, <= 65536) to
 * MXFP4: codes uint8 [rows][K/2], scales uint8 [rows][K/32]. Per block of 32:
 * X = 2^(floor(log2 max|v|) - 2), the exponent clamped to [-127, 127]
 * (an all-zero block gets s = 0); each v / X rounded to the nearest E2M1
 * magnitude, ties to the even code, magnitudes past 6 held at 6, the sign of
 * v kept. Bit-exact (every decision is taken on the exact binary32 value).
 */
moe_status moe_mxfp4_quantize(int64_t rows, int32_t K, const uint16_t *x, uint8_t *codes, uint8_t *scales,
                              void *stream);

/*
 * Grouped GEMM on MXFP4 operands, the same row semantics as
 * moe_grouped_gemm_w4a16: for local expert e and rows r in
 * [offsets[e], offsets[e+1]) the activation row is row a_row_index[r] / top_k
 * of (a_codes [T][K/2], a_scales [T][K/32]) when a_row_index != NULL, else
 * row r of (a_codes [T*k][K/2], a_scales [T*k][K/32]). Kinds and outputs as
 * moe_grouped_gemm_w4a16 (W13_SWIGLU: bf16 h = silu(g) * u; W2 / W13_RAW: bf16
 * or f32). Accumulation is binary32 in the matrix unit over exact FP4 products
 * with power-of-two block scales. No workspace.
 */
moe_status moe_grouped_gemm_mxfp4(const moe_shape *shape, moe_gemm_kind kind, const uint8_t *a_codes,
                                  const uint8_t *a_scales, const int32_t *a_row_index, const int32_t *offsets,
                                  const uint8_t *wq, const uint8_t *ws, void *c, moe_dtype c_dtype, void *stream);

/*
 * Reorder one MXFP4 weight matrix's codes from the plain layout into the
 * tiled MXFP4 layout above (for callers whose weights are fixed: each code
 * load of the GEMMs then reads 1 KiB contiguously). Arguments and errors as
 * moe_w4a16_pack_weights, with an MXFP4 shape (group_size 32;
 * weight_layout is ignored). Bit-exact byte permutation.
 */
moe_status moe_mxfp4_pack_weights(const moe_shape *shape, moe_gemm_kind kind, const uint8_t *wq, uint8_t *wq_tiled,
                                  void *stream);

/*
 * The W4A4 layer: route -> permute -> quantize x (per token, 32 along H) ->
 * gate/up GEMM (h = bf16(silu(g) * u)) -> requantize h (32 along I) -> down
 * GEMM (y bf16) -> finalize (the W4A16 layer's combine). Arguments as
 * moe_w4a16_forward with MXFP4 weights; workspace >= moe_w4a4_workspace_size
 * bytes (0 for an invalid shape), 256-B aligned.
 */
size_t moe_w4a4_workspace_size(const moe_shape *shape);
moe_status moe_w4a4_forward(const moe_shape *shape, const uint16_t *x, const float *router_logits,
                            const uint8_t *w13_q, const uint8_t *w13_s, const uint8_t *w2_q, const uint8_t *w2_s,
                            uint16_t *out, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Launch-shape override, for tests and tuning (not a passage of the pages: a
 * switch over this library's own kernel variants). Every field -1 keeps the
 * automatic choice. A field changes which kernel variant runs and how it
 * tiles the work, never a result: the variants compute the same bits, which
 * the tests check by forcing each one. Process-wide; set it from one thread
 * while no other call is being issued. NULL resets every field to -1. Values
 * a kernel does not support fall back to a supported variant. Returns MOE_OK.
 */
typedef struct {
    int32_t gemm_mode;                   /* grouped GEMM kernel: 0 split-K, 1 streaming,
                                            2 tile kernel (8 waves, 64-row chunks),
                                            3 tile kernel (4 waves, 32-row chunks)      */
    int32_t gemm_tiles_per_wave;         /* streaming: 16-row weight tiles per wave     */
    int32_t gemm_subtiles;               /* streaming: 16-token subtiles per chunk      */
    int32_t gemm_kseg;                   /* streaming: 128-wide groups per K segment    */
    int32_t gemm_ring;                   /* streaming: weight register ring depth       */
    int32_t gemm_nontemporal;            /* streaming: 1 non-temporal code loads, 0 not */
    int32_t permute_parallel_min_tokens; /* permute over token ranges past this T       */
    int32_t route_fuse_max_tokens;       /* layer routes inside the permute up to this T */
    int32_t decode_max_tokens;           /* layer takes the small-batch path up to this T
                                            (routing inside the gate/up GEMM; 0: never) */
    int32_t decode_combine_max_tokens;   /* small-batch path: down GEMM and combine in one
                                            launch up to this T (0: never)              */
    int32_t perm_in_gemm_max_tokens;     /* general path: the gate/up GEMM builds the
                                            permutation from the routing ids up to this T
                                            (no permutation launch; 0: never)           */
} moe_launch_override;

moe_status moe_w4a16_set_launch_override(const moe_launch_override *ov);

#ifdef __cplusplus
}
#endif

#endif /* MOE_W4A16_H */

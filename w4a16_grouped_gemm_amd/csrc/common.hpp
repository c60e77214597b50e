// common.hpp -- shared device helpers and the internal launcher interface of
// the gfx950 W4A16 MoE library. Everything here is gfx950-only HIP.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe_w4a16.h"

namespace moe {

constexpr int kGroup = 128;          // quantisation group along K
constexpr int kMaxExperts = 1024;    // E_g and E_loc limit (LDS tables)
constexpr int kMaxSharedExperts = 4; // shared experts of one layer call; the grouped GEMMs then
                                     // see up to kMaxExperts + kMaxSharedExperts experts
constexpr int kMaxTopK = 16;
constexpr int kMaxDim = 16384;       // H and I limit
constexpr int kMaxTokens = 1 << 18;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// binary32 -> bf16, round to nearest even on the bit pattern (exact for
// normals, subnormals and overflow; bf16 shares binary32's exponent range so
// there is nothing to flush). NaN -> quiet NaN with the same sign.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u)
        return (u >> 16) | 0x0040u;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

// Wave-level (64-lane) exclusive prefix sum of an int; also returns the total.
__device__ __forceinline__ int wave_exclusive_scan(int v, int &total)
{
    // inclusive scan in registers: row_shr 1, 2, 4, 8 within each 16-lane
    // row (lanes shifted in from outside the row add 0), then row_bcast:15
    // adds each row's last lane to the next row (rows 1 and 3) and
    // row_bcast:31 adds lane 31 to rows 2 and 3
    int x = v;
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);
    total = __builtin_amdgcn_readlane(x, 63);
    return x - v;
}

// ---- launchers (host side, one per kernel family) ------------------------

struct GemmLaunch {
    moe_gemm_kind kind;
    const uint16_t *a;
    const int32_t *a_row_index;
    int top_k;
    const int32_t *offsets;   // NULL: one dense expert with dense_rows rows
    int dense_rows;
    int num_experts;          // E_loc
    const uint8_t *wq;
    const uint16_t *s;
    const uint8_t *wq_sh;     // NULL, or the shared experts (experts e_routed.. of the launch)
    const uint16_t *s_sh;
    int e_routed;
    void *c;
    const int32_t *c_row_index;  // NULL, or row r of the result is stored at row c_row_index[r]
    bool c_f32;
    int K;                    // reduction length
    int N;                    // weight rows per expert
    int max_rows;             // T * k: upper bound on R
    int expected_rows;        // expected R (routed slots on local experts)
    size_t a_bytes;           // bytes of the activation array `a`
    bool w_tiled;             // codes in the tiled layout (1 KiB per tile and group)
};

// x non-NULL (the W4A4 layer): the launch also quantizes x [T][H] to MXFP4
// codes xq [T][H/2] and scales xs [T][H/32] (the quantize kernel's bits)
hipError_t launch_route(const moe_shape &sh, const float *logits, int32_t *ids, float *w,
                        hipStream_t st, const uint16_t *x = nullptr, uint8_t *xq = nullptr,
                        uint8_t *xs = nullptr);
// part: workspace of permute_workspace_bytes(sh) (the per-range counts of
// the parallel path for many tokens; NULL when that size is 0)
hipError_t launch_permute(const moe_shape &sh, const int32_t *ids, int32_t *counts,
                          int32_t *offsets, int32_t *perm, int32_t *inv_perm, hipStream_t st,
                          int num_shared = 0, int32_t *part = nullptr);
size_t permute_workspace_bytes(const moe_shape &sh);
bool route_permute_fusable(const moe_shape &sh);
hipError_t launch_route_permute(const moe_shape &sh, const float *logits, int32_t *ids, float *w,
                                int32_t *counts, int32_t *offsets, int32_t *perm, int32_t *inv_perm,
                                hipStream_t st,
                                int num_shared = 0, const uint16_t *x = nullptr, uint8_t *xq = nullptr,
                                uint8_t *xs = nullptr);
hipError_t launch_gather(const moe_shape &sh, const uint16_t *x, const int32_t *perm,
                         const int32_t *offsets, uint16_t *x_perm, hipStream_t st);
hipError_t launch_grouped_gemm(const GemmLaunch &g, hipStream_t st);
// The layer's gate/up GEMM with the permutation built inside it from the
// routing ids (no permutation launch): g as for launch_grouped_gemm with
// a_row_index unused; the permutation's tables (as moe_permute stores them)
// go to the IdsSource outputs.
constexpr int kDecMaxSlots = 128;                   // T * k of the layers' small-batch paths

struct IdsSource {
    const int32_t *ids;       // [T*k] global expert ids
    int T, begin;             // tokens; global id of local expert 0
    int32_t *counts, *offsets, *perm, *inv_perm;
};
bool gemm_ids_supported(const GemmLaunch &g, int T);
hipError_t launch_gemm_ids(const GemmLaunch &g, const IdsSource &src, hipStream_t st);
hipError_t launch_pack_weights(int E, int N, int K, int half, bool pair_rows, const uint8_t *wq,
                               uint8_t *wq_tiled, hipStream_t st, bool shuffle = true);
hipError_t launch_finalize(const moe_shape &sh, const void *y, bool y_f32, const float *w,
                           const int32_t *inv_perm, void *out, bool out_f32, hipStream_t st,
                           bool y_slot = false, int num_shared = 0,
                           const int32_t *shared_row0 = nullptr);

// The grouped GEMM's launch choice for a shape: kernel family (0 split-K,
// 1 streaming, 2 / 3 tile kernel) and the streaming tiling. The families
// sum in different orders; within a family every tiling gives the same bits.
struct LaunchChoice {
    int mode, tpw, nsub, kseg, ring;
    bool nt;
};
LaunchChoice choose_launch(const GemmLaunch &g);
GemmLaunch layer_gemm_args(const moe_shape &sh, moe_gemm_kind kind);

// Item source of the small-batch path on the streaming kernel: src 1 routes
// inside the kernel (gate/up; writes ids / w / pres), src 2 reads the stored
// slot table (down). T tokens, E_g logit columns, local experts from begin.
struct DecodeSource {
    int src;
    const float *logits;
    int T, E_g, begin;
    int32_t *ids;
    float *w;
    int32_t *pres;
};
hipError_t launch_decode_stream(const GemmLaunch &g, const DecodeSource &d, hipStream_t st);
bool decode_stream_supported(const GemmLaunch &g);

// The layer's small-batch path (decode.hip): up to 16 tokens, no shared
// experts, E_g <= 256. h and y are in slot order; pres[t*k + j] is the slot
// index when the slot's expert is local, else -1.
bool decode_path_fits(const moe_shape &sh, int num_shared);
bool decode_combine_fits(const moe_shape &sh);
hipError_t launch_decode_gate_up(const moe_shape &sh, const float *logits, const uint16_t *x, const uint8_t *w13,
                                 const uint16_t *s13, int32_t *ids, float *w, int32_t *pres, uint16_t *h,
                                 hipStream_t st);
hipError_t launch_decode_down(const moe_shape &sh, const int32_t *ids, const int32_t *pres, const uint16_t *h,
                              const uint8_t *w2, const uint16_t *s2, uint16_t *y, hipStream_t st);
hipError_t launch_decode_down_combine(const moe_shape &sh, const int32_t *ids, const float *w, const int32_t *pres,
                                      const uint16_t *h, const uint8_t *w2, const uint16_t *s2, uint16_t *out,
                                      hipStream_t st);

// The W4A4 variant (gemm_mxfp4.hip): MXFP4 operands, E8M0 scale per 32 along K.
struct MxGemmLaunch {
    moe_gemm_kind kind;
    const uint8_t *a;            // activation codes [a_rows][K/2]
    const uint8_t *as;           // activation scales [a_rows][K/32]
    const int32_t *a_row_index;  // NULL, or row r reads activation row a_row_index[r] / top_k
    long long a_rows;
    int top_k;
    const int32_t *offsets;      // [E+1] on the device
    int num_experts;
    const uint8_t *wq;           // [E][N][K/2]
    const uint8_t *ws;           // [E][N][K/32]
    void *c;
    const int32_t *c_row_index;  // NULL, or result row r is stored at row c_row_index[r]
    bool c_f32;
    int K, N;
    int max_rows, expected_rows;
    bool w_tiled;                // codes in the tiled layout (scales plain)
    // SwiGLU only, non-NULL: h also stored requantized to MXFP4 ([max_rows][N/4]
    // codes, [max_rows][N/64] scales; the routed rows, counted on the device);
    // c is then scratch for bf16 h
    uint8_t *cq, *cs;
    // non-NULL: the permutation is built inside the GEMM from these routing
    // ids ([T*k], global expert ids; offsets and a_row_index unused) and its
    // tables (as moe_permute stores them) go to the outputs below
    const int32_t *ids;
    int T, begin;
    int32_t *counts_out, *offsets_out, *perm_out, *inv_perm_out;
};
hipError_t launch_mx_grouped_gemm(const MxGemmLaunch &g, hipStream_t st);
bool mx_gemm_ids_supported(const MxGemmLaunch &g, int T);
// The W4A4 layer's small-batch path (T * k <= 128): the gate/up GEMM routes
// the tokens itself (logits non-NULL: writes ids, w, pres) and quantizes
// their x rows while staging them, its outputs h rows t*k + j (requantized,
// g.cq / g.cs); the down GEMM (logits NULL) reads that stored slot table and
// writes y rows t*k + j. g as for launch_mx_grouped_gemm (offsets,
// a_row_index, c_row_index unused).
struct MxSmallSource {
    const float *logits;      // [T][E_g] (gate/up) or NULL (down)
    int E_g, T, begin;
    const uint16_t *x;        // bf16 x [T][H] (gate/up)
    int32_t *ids;             // [T*k] global expert ids
    float *w;                 // [T*k] routing weights
    int32_t *pres;            // [T*k] slot if local, else -1
};
bool mx_small_supported(const MxGemmLaunch &g);
hipError_t launch_mx_small(const MxGemmLaunch &g, const MxSmallSource &src, hipStream_t st);
// rows_dev (nullable): the device-side row count to quantize (at most rows)
hipError_t launch_mx_quantize(long long rows, int K, const uint16_t *x, uint8_t *codes, uint8_t *scales,
                              const int32_t *rows_dev, hipStream_t st);

int device_cu_count();

// Process-wide launch-shape override (moe_w4a16_set_launch_override); every
// field -1 = automatic. Only which kernel runs and its tiling depend on it.
moe_launch_override launch_override();

}  // namespace moe

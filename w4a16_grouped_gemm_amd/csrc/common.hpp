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

hipError_t launch_route(const moe_shape &sh, const float *logits, int32_t *ids, float *w,
                        hipStream_t st);
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
                                int num_shared = 0);
hipError_t launch_gather(const moe_shape &sh, const uint16_t *x, const int32_t *perm,
                         const int32_t *offsets, uint16_t *x_perm, hipStream_t st);
hipError_t launch_grouped_gemm(const GemmLaunch &g, hipStream_t st);
hipError_t launch_pack_weights(int E, int N, int K, int half, bool pair_rows, const uint8_t *wq,
                               uint8_t *wq_tiled, hipStream_t st);
hipError_t launch_finalize(const moe_shape &sh, const void *y, bool y_f32, const float *w,
                           const int32_t *inv_perm, void *out, bool out_f32, hipStream_t st,
                           bool y_slot = false, int num_shared = 0,
                           const int32_t *shared_row0 = nullptr);

int device_cu_count();

}  // namespace moe

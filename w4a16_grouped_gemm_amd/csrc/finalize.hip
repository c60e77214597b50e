// finalize.hip -- weighted unpermute / combine of the expert outputs.
//
// FlashInfer PR #7196 analysis, section 1 (`moe_finalize.py`): per output
// element the first slot is a plain fp32 multiply (so a signed zero survives),
// every later slot an fp32 FMA in slot order, and the FMA no longer flushes
// subnormals to zero; section 2 ("Arithmetic Alignment") restates the order.
// InfiniLM PR #500 report, section 2.2 scatters with index_add_ atomics, which
// its section 3 blames for run-to-run differences; here the combine is a
// gather over the token's slots instead, so it is deterministic.
//
// gfx950 notes: this file is compiled without FP contraction and with fp32
// denormals preserved (the kernel descriptor's f32 denorm mode is "keep"),
// so v_mul_f32 / v_fma_f32 are exactly IEEE binary32 multiply / FMA with
// round-to-nearest-even. One thread owns 8 consecutive columns of one token:
// 16-byte (bf16) or 2x16-byte (fp32) coalesced row loads per slot, all of a
// token's slots in flight at once.
#include "common.hpp"

namespace moe {

namespace {

// KMAX >= k. All of a token's row indices and weights are read first, then
// all of its expert rows, so a thread waits for two memory round trips
// instead of two per slot; the combine then runs in slot order.
// Y_SLOT: y is in slot order (row t*k + j, as the layer's down GEMM writes
// it when every slot is local), so the row loads need no index and go out
// together with the index and weight loads: one round trip. inv_perm then
// only says which slots are present.
// SHARED: the layer's shared experts (GC-MoE abstract: optional shared
// experts): nsh <= kMaxShared rows per token at y row R + s*T + t, R =
// *shared_row0 (the routed row count), each added with weight 1 after the
// routed slots: acc = acc + v, or v as the token's first term.
constexpr int kMaxShared = kMaxSharedExperts;

template <bool Y_F32, bool OUT_F32, int KMAX, bool Y_SLOT, bool SHARED>
__global__ __launch_bounds__(256) void finalize_kernel(int T, int k, int H,
                                                       const void *__restrict__ y,
                                                       const float *__restrict__ w,
                                                       const int32_t *__restrict__ inv,
                                                       void *__restrict__ out, int nsh,
                                                       const int32_t *__restrict__ shared_row0)
{
    const int R0 = SHARED ? shared_row0[0] : 0;
    const int vec_per_row = H >> 3;
    const long long total = (long long)T * vec_per_row;
    for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (long long)gridDim.x * blockDim.x) {
        const int t = (int)(i / vec_per_row);
        const int c0 = (int)(i - (long long)t * vec_per_row) * 8;
        // No load below sits under a branch (a load under one makes the
        // compiler wait for every earlier load first, serialising the round
        // trips): slots past k re-read slot k - 1, absent slots read row 0,
        // and both are masked in the combine.
        int32_t r[KMAX];
        float wt[KMAX];
#pragma unroll
        for (int j = 0; j < KMAX; ++j) {
            const size_t sl = (size_t)t * k + (j < k ? j : k - 1);
            r[j] = inv[sl];
            wt[j] = w[sl];
        }
        float v[KMAX][8];
#pragma unroll
        for (int j = 0; j < KMAX; ++j) {
            const size_t yrow = Y_SLOT ? (size_t)t * k + (j < k ? j : k - 1) : (size_t)(r[j] >= 0 ? r[j] : 0);
            if (Y_F32) {
                const float *src = static_cast<const float *>(y) + yrow * H + c0;
                const floatx4 a = *reinterpret_cast<const floatx4 *>(src);
                const floatx4 b = *reinterpret_cast<const floatx4 *>(src + 4);
                v[j][0] = a.x; v[j][1] = a.y; v[j][2] = a.z; v[j][3] = a.w;
                v[j][4] = b.x; v[j][5] = b.y; v[j][6] = b.z; v[j][7] = b.w;
            } else {
                const uint16_t *src = static_cast<const uint16_t *>(y) + yrow * H + c0;
                const u32x4 d = *reinterpret_cast<const u32x4 *>(src);
                v[j][0] = bf16_to_f32(d.x & 0xFFFFu); v[j][1] = bf16_to_f32(d.x >> 16);
                v[j][2] = bf16_to_f32(d.y & 0xFFFFu); v[j][3] = bf16_to_f32(d.y >> 16);
                v[j][4] = bf16_to_f32(d.z & 0xFFFFu); v[j][5] = bf16_to_f32(d.z >> 16);
                v[j][6] = bf16_to_f32(d.w & 0xFFFFu); v[j][7] = bf16_to_f32(d.w >> 16);
            }
        }
#pragma unroll
        for (int j = 0; j < KMAX; ++j)
            if (j >= k)
                r[j] = -1;
        float vs[SHARED ? kMaxShared : 1][8];
        if (SHARED) {
#pragma unroll
            for (int sh = 0; sh < kMaxShared; ++sh) {
                // every row is loaded (clamped to the last shared expert), no branch
                const size_t row = (size_t)R0 + (size_t)(sh < nsh ? sh : nsh - 1) * T + t;
                const uint16_t *src = static_cast<const uint16_t *>(y) + row * H + c0;
                const u32x4 d = *reinterpret_cast<const u32x4 *>(src);
                vs[sh][0] = bf16_to_f32(d.x & 0xFFFFu); vs[sh][1] = bf16_to_f32(d.x >> 16);
                vs[sh][2] = bf16_to_f32(d.y & 0xFFFFu); vs[sh][3] = bf16_to_f32(d.y >> 16);
                vs[sh][4] = bf16_to_f32(d.z & 0xFFFFu); vs[sh][5] = bf16_to_f32(d.z >> 16);
                vs[sh][6] = bf16_to_f32(d.w & 0xFFFFu); vs[sh][7] = bf16_to_f32(d.w >> 16);
            }
        }
        float acc[8];
#pragma unroll
        for (int q = 0; q < 8; ++q)
            acc[q] = 0.0f;
        bool first = true;
#pragma unroll
        for (int j = 0; j < KMAX; ++j) {
            if (r[j] < 0)
                continue;
            if (first) {
#pragma unroll
                for (int q = 0; q < 8; ++q)
                    acc[q] = __fmul_rn(v[j][q], wt[j]);
                first = false;
            } else {
#pragma unroll
                for (int q = 0; q < 8; ++q)
                    acc[q] = __fmaf_rn(v[j][q], wt[j], acc[q]);
            }
        }
        if (SHARED) {
#pragma unroll
            for (int sh = 0; sh < kMaxShared; ++sh) {
                if (sh >= nsh)
                    break;
#pragma unroll
                for (int q = 0; q < 8; ++q)
                    acc[q] = first ? vs[sh][q] : __fadd_rn(acc[q], vs[sh][q]);
                first = false;
            }
        }
        if (OUT_F32) {
            float *dst = static_cast<float *>(out) + (size_t)t * H + c0;
            *reinterpret_cast<floatx4 *>(dst) = floatx4{acc[0], acc[1], acc[2], acc[3]};
            *reinterpret_cast<floatx4 *>(dst + 4) = floatx4{acc[4], acc[5], acc[6], acc[7]};
        } else {
            uint16_t *dst = static_cast<uint16_t *>(out) + (size_t)t * H + c0;
            *reinterpret_cast<u32x4 *>(dst) =
                u32x4{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                      pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7])};
        }
    }
}

template <bool Y_F32, bool OUT_F32, bool Y_SLOT, bool SHARED = false>
void launch_fin(dim3 grid, dim3 block, hipStream_t st, int T, int k, int H, const void *y, const float *w,
                const int32_t *inv, void *out, int nsh = 0, const int32_t *r0 = nullptr)
{
    if (k <= 2)
        hipLaunchKernelGGL((finalize_kernel<Y_F32, OUT_F32, 2, Y_SLOT, SHARED>), grid, block, 0, st, T, k, H, y, w,
                           inv, out, nsh, r0);
    else if (k <= 4)
        hipLaunchKernelGGL((finalize_kernel<Y_F32, OUT_F32, 4, Y_SLOT, SHARED>), grid, block, 0, st, T, k, H, y, w,
                           inv, out, nsh, r0);
    else if (k <= 8)
        hipLaunchKernelGGL((finalize_kernel<Y_F32, OUT_F32, 8, Y_SLOT, SHARED>), grid, block, 0, st, T, k, H, y, w,
                           inv, out, nsh, r0);
    else
        hipLaunchKernelGGL((finalize_kernel<Y_F32, OUT_F32, kMaxTopK, Y_SLOT, SHARED>), grid, block, 0, st, T, k, H,
                           y, w, inv, out, nsh, r0);
}

}  // namespace

hipError_t launch_finalize(const moe_shape &sh, const void *y, bool y_f32, const float *w,
                           const int32_t *inv_perm, void *out, bool out_f32, hipStream_t st, bool y_slot,
                           int num_shared, const int32_t *shared_row0)
{
    const long long total = (long long)sh.num_tokens * (sh.hidden / 8);
    long long blocks = (total + 255) / 256;
    const long long cap = (long long)device_cu_count() * 32;
    if (blocks > cap)
        blocks = cap;
    if (blocks < 1)
        blocks = 1;
    const dim3 grid((unsigned)blocks), block(256);
    const int T = sh.num_tokens, k = sh.top_k, H = sh.hidden;
    if (num_shared > 0)                           // the layer with shared experts: bf16 y and out
        launch_fin<false, false, false, true>(grid, block, st, T, k, H, y, w, inv_perm, out, num_shared,
                                              shared_row0);
    else if (y_slot)                              // the layer's path: bf16 y in slot order, bf16 out
        launch_fin<false, false, true>(grid, block, st, T, k, H, y, w, inv_perm, out);
    else if (y_f32 && out_f32)
        launch_fin<true, true, false>(grid, block, st, T, k, H, y, w, inv_perm, out);
    else if (y_f32)
        launch_fin<true, false, false>(grid, block, st, T, k, H, y, w, inv_perm, out);
    else if (out_f32)
        launch_fin<false, true, false>(grid, block, st, T, k, H, y, w, inv_perm, out);
    else
        launch_fin<false, false, false>(grid, block, st, T, k, H, y, w, inv_perm, out);
    return hipGetLastError();
}

}  // namespace moe

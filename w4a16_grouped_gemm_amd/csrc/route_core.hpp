// route_core.hpp -- per-token top-k selection and renormalised weights,
// shared by the routing kernel and the fused routing + permutation kernel.
//
// Layer definition: softmax over all experts, keep the top-k, renormalise; the
// i-th selected expert is slot i (FlashInfer PR #7196 analysis, section 2:
// the combine walks slots "first slot, then in order"). Because softmax is
// monotone the selection runs on the logits; because the normaliser over all
// experts cancels in the renormalisation, weight i is
// exp(l_i - l_0) / sum_{j<k} exp(l_j - l_0).
#pragma once

#include "common.hpp"

namespace moe {

// Monotone map of a binary32 to uint32 (total order for non-NaN values).
__device__ __forceinline__ uint32_t ordered_bits(float v)
{
    if (v == 0.0f)
        v = 0.0f;                          // -0 == +0
    uint32_t u = __float_as_uint(v);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inverse of ordered_bits (a -0 logit comes back as +0, which exp treats alike).
__device__ __forceinline__ float from_ordered_bits(uint32_t o)
{
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

// Cross-lane max / min over the 16 lanes of a DPP row, every lane ending
// with the result: xor-1 and xor-2 quad permutes, then the half-row and row
// mirrors (each step pairs disjoint lane sets, so after four steps every lane
// has seen all sixteen).
template <bool MAX>
__device__ __forceinline__ uint32_t row_reduce(uint32_t v)
{
    const int id = MAX ? 0 : -1;          // identity for lanes a DPP read cannot reach
#define MOE_DPP_STEP(ctrl)                                                              \
    {                                                                                   \
        const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, ctrl, 0xF, 0xF, false); \
        v = MAX ? (o > v ? o : v) : (o < v ? o : v);                                    \
    }
    MOE_DPP_STEP(0xB1)     // quad_perm [1,0,3,2]
    MOE_DPP_STEP(0x4E)     // quad_perm [2,3,0,1]
    MOE_DPP_STEP(0x141)    // row_half_mirror
    MOE_DPP_STEP(0x140)    // row_mirror
#undef MOE_DPP_STEP
    return v;
}

// Reduction over the TL lanes that hold one token (TL = 16: a DPP row;
// TL = 64: the four rows of the wave combined through readlane).
template <int TL, bool MAX>
__device__ __forceinline__ uint32_t token_reduce(uint32_t v)
{
    v = row_reduce<MAX>(v);
    if (TL == 64) {
        uint32_t r = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
#pragma unroll
        for (int q = 1; q < 4; ++q) {
            const uint32_t o = (uint32_t)__builtin_amdgcn_readlane((int)v, 16 * q);
            r = MAX ? (o > r ? o : r) : (o < r ? o : r);
        }
        v = r;
    }
    return v;
}

// One token held by TL lanes (q = lane within the token, PL logits per lane,
// E <= TL * PL). Each of the k rounds takes the largest remaining ordered
// logit over the token's lanes, then the lowest expert index holding it, and
// retires that expert; ordered value 0 marks a retired or absent expert (no
// non-NaN logit maps to 0). Lane q == j ends with slot j's expert and weight.
template <int TL, int PL>
__device__ __forceinline__ void route_token(const float *__restrict__ row, int E, int k, int q, int &e_out,
                                            float &w_out)
{
    // every load is issued (a clamped index, no branch), so the PL loads
    // are one memory round trip; entries past E are masked afterwards
    float lv[PL];
#pragma unroll
    for (int i = 0; i < PL; ++i) {
        const int e = q + TL * i;
        lv[i] = row[e < E ? e : E - 1];
    }
    uint32_t val[PL];
#pragma unroll
    for (int i = 0; i < PL; ++i)
        val[i] = q + TL * i < E ? ordered_bits(lv[i]) : 0u;
    float l0 = 0.0f;                                   // the largest logit (slot 0)
    float my_v = 0.0f;                                 // lane q < k: logit of slot q
    int my_e = -1;                                     // lane q < k: expert of slot q
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
        if (j >= k)
            break;
        uint32_t bv = 0;
#pragma unroll
        for (int i = 0; i < PL; ++i)
            bv = val[i] > bv ? val[i] : bv;
        uint32_t m;
        int e;
        if constexpr (TL == 64) {
            // whole wave: each row's maximum, then rows 1 and 3 take lane
            // 15's and 47's, rows 2 and 3 lane 31's (DPP row broadcasts), so
            // lane 63 holds the wave's maximum: one readlane instead of four
            bv = row_reduce<true>(bv);
            uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)bv, 0x142, 0xA, 0xF, false);   // row_bcast:15
            bv = o > bv ? o : bv;
            o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)bv, 0x143, 0xC, 0xF, false);            // row_bcast:31
            bv = o > bv ? o : bv;
            m = (uint32_t)__builtin_amdgcn_readlane((int)bv, 63);
            // lowest index holding m: indices q + 64 i ascend with i, then with
            // the lane, so the first i whose ballot is not empty decides
            e = -1;
#pragma unroll
            for (int i = PL - 1; i >= 0; --i) {
                const uint64_t b = __ballot(val[i] == m);
                if (b)
                    e = 64 * i + __builtin_ctzll(b);
            }
        } else {
            m = token_reduce<TL, true>(bv);
            uint32_t bi = 0xFFFFFFFFu;
#pragma unroll
            for (int i = PL - 1; i >= 0; --i)           // lowest index of this lane holding m
                bi = val[i] == m ? (uint32_t)(q + TL * i) : bi;
            e = (int)token_reduce<TL, false>(bi);
        }
        if (j == 0)
            l0 = from_ordered_bits(m);
        if (q == j) {
            my_e = e;
            my_v = from_ordered_bits(m);
        }
        // the owner lane retires the winner
#pragma unroll
        for (int i = 0; i < PL; ++i)
            if (q + TL * i == e)
                val[i] = 0u;
    }
    // renormalised softmax over the k selected logits (fp32), one slot per
    // lane. The difference l_q - l_0 is formed error-free (TwoSum: d + r ==
    // l_q - l_0 exactly) and exp(d + r) ~= exp(d) * (1 + r), so wide logit
    // ranges lose no accuracy before the exponential. The normaliser is a
    // DPP row sum over the 16 lanes holding the slots (k <= 16; lanes q >= k
    // add 0); every lane of the row ends with the same sum.
    // A slot whose difference is not finite (a -inf logit, i.e. a masked
    // expert, or l_q - l_0 overflowing to -inf) has exp(d) = 0 exactly; the
    // correction term is then NaN (inf - inf) and is not applied.
    float ex = 0.0f;
    if (q < k) {
        const float a = my_v, b = -l0;
        const float d = a + b;
        const float ap = d - b;
        const float bp = d - ap;
        const float r = (a - ap) + (b - bp);
        const float ed = expf(d);
        ex = __builtin_isfinite(d) ? __builtin_fmaf(ed, r, ed) : ed;
    }
    float z = ex;
#define MOE_DPP_ADD(ctrl) z += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(z), ctrl, 0xF, 0xF, false));
    MOE_DPP_ADD(0xB1)      // quad_perm [1,0,3,2]
    MOE_DPP_ADD(0x4E)      // quad_perm [2,3,0,1]
    MOE_DPP_ADD(0x141)     // row_half_mirror
    MOE_DPP_ADD(0x140)     // row_mirror
#undef MOE_DPP_ADD
    e_out = q < k ? my_e : -1;
    w_out = q < k ? ex / z : 0.0f;
}

}  // namespace moe

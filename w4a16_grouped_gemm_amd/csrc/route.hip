// route.hip -- wavefront-level top-k routing with softmax renormalisation.
//
// Layer definition: softmax over all experts, keep the top-k, renormalise; the
// i-th selected expert is slot i (FlashInfer PR #7196 analysis, section 2:
// the combine walks slots "first slot, then in order"). Because softmax is
// monotone the selection runs on the logits; because the normaliser over all
// experts cancels in the renormalisation, weight i is
// exp(l_i - l_0) / sum_{j<k} exp(l_j - l_0).
//
// 16 lanes per token (a DPP row) for E <= 256, a whole wave for larger E;
// lane q holds logits q, q+TL, ... . Each of k rounds takes the largest
// remaining logit (on an order-preserving integer image; -0 is folded to +0
// so equal logits tie exactly as IEEE equality says), then the lowest expert
// index holding it: the order (logit desc, index asc).
#include "common.hpp"

namespace moe {

namespace {

constexpr int kRouteWaves = 4;

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

// TL lanes per token, PL logits per lane (E <= TL * PL). Each of the k rounds
// takes the largest remaining ordered logit over the token's lanes, then the
// lowest expert index holding it, and retires that expert; ordered value 0
// marks a retired or absent expert (no non-NaN logit maps to 0).
template <int TL, int PL>
__global__ __launch_bounds__(kRouteWaves * 64) void route_kernel(int T, int E, int k,
                                                                 const float *__restrict__ logits,
                                                                 int32_t *__restrict__ ids,
                                                                 float *__restrict__ w)
{
    constexpr int TPW = 64 / TL;                       // tokens per wave
    const int lane = threadIdx.x & 63;
    const int q = lane % TL;                           // lane within the token
    const int t = (blockIdx.x * kRouteWaves + (threadIdx.x >> 6)) * TPW + lane / TL;
    if (t >= T)
        return;
    const float *row = logits + (size_t)t * E;
    uint32_t val[PL];
#pragma unroll
    for (int i = 0; i < PL; ++i) {
        const int e = q + TL * i;
        val[i] = e < E ? ordered_bits(row[e]) : 0u;
    }
    float sel_v[kMaxTopK];
    int sel_e[kMaxTopK];
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
        if (j >= k)
            break;
        uint32_t bv = 0;
#pragma unroll
        for (int i = 0; i < PL; ++i)
            bv = val[i] > bv ? val[i] : bv;
        const uint32_t m = token_reduce<TL, true>(bv);
        uint32_t bi = 0xFFFFFFFFu;
#pragma unroll
        for (int i = PL - 1; i >= 0; --i)               // lowest index of this lane holding m
            bi = val[i] == m ? (uint32_t)(q + TL * i) : bi;
        const int e = (int)token_reduce<TL, false>(bi);
        sel_e[j] = e;
        sel_v[j] = from_ordered_bits(m);
        // the owner lane retires the winner
#pragma unroll
        for (int i = 0; i < PL; ++i)
            if (q + TL * i == e)
                val[i] = 0u;
    }
    // renormalised softmax over the k selected logits (fp32). The difference
    // l_j - l_0 is formed error-free (TwoSum: d + r == l_j - l_0 exactly) and
    // exp(d + r) ~= exp(d) * (1 + r), so wide logit ranges lose no accuracy
    // before the exponential.
    const float l0 = sel_v[0];
    float z = 0.0f;
    float ex[kMaxTopK];
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
        if (j >= k)
            break;
        const float a = sel_v[j], b = -l0;
        const float d = a + b;
        const float ap = d - b;
        const float bp = d - ap;
        const float r = (a - ap) + (b - bp);
        const float e = expf(d);
        ex[j] = __builtin_fmaf(e, r, e);
        z += ex[j];
    }
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
        if (j >= k)
            break;
        if (q == j) {
            ids[(size_t)t * k + j] = sel_e[j];
            w[(size_t)t * k + j] = ex[j] / z;
        }
    }
}

}  // namespace

hipError_t launch_route(const moe_shape &sh, const float *logits, int32_t *ids, float *w,
                        hipStream_t st)
{
    const int T = sh.num_tokens;
    const int E = sh.num_experts;
    const int k = sh.top_k;
    const dim3 block(kRouteWaves * 64);
    auto grid = [&](int tl) { return dim3((T + kRouteWaves * (64 / tl) - 1) / (kRouteWaves * (64 / tl))); };
    if (E <= 64 && k <= 16)
        hipLaunchKernelGGL((route_kernel<16, 4>), grid(16), block, 0, st, T, E, k, logits, ids, w);
    else if (E <= 128 && k <= 16)
        hipLaunchKernelGGL((route_kernel<16, 8>), grid(16), block, 0, st, T, E, k, logits, ids, w);
    else if (E <= 256 && k <= 16)
        hipLaunchKernelGGL((route_kernel<16, 16>), grid(16), block, 0, st, T, E, k, logits, ids, w);
    else if (E <= 512)
        hipLaunchKernelGGL((route_kernel<64, 8>), grid(64), block, 0, st, T, E, k, logits, ids, w);
    else
        hipLaunchKernelGGL((route_kernel<64, kMaxExperts / 64>), grid(64), block, 0, st, T, E, k, logits, ids, w);
    return hipGetLastError();
}

}  // namespace moe

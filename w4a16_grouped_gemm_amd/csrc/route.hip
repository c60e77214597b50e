// route.hip -- wavefront-level top-k routing with softmax renormalisation.
//
// Layer definition: softmax over all experts, keep the top-k, renormalise; the
// i-th selected expert is slot i (FlashInfer PR #7196 analysis, section 2:
// the combine walks slots "first slot, then in order"). Because softmax is
// monotone the selection runs on the logits; because the normaliser over all
// experts cancels in the renormalisation, weight i is
// exp(l_i - l_0) / sum_{j<k} exp(l_j - l_0).
//
// One 64-lane wavefront per token; lane L holds logits L, L+64, ... (E <= 1024
// -> at most 16 per lane). k rounds of a wave arg-max on a 64-bit key that
// orders (logit desc, index asc); -0 is folded to +0 so equal logits tie on
// the index exactly as IEEE equality says.
#include "common.hpp"

namespace moe {

namespace {

constexpr int kRouteWaves = 4;
constexpr int kPerLane = kMaxExperts / 64;

// Monotone map of a binary32 to uint32 (total order for non-NaN values).
__device__ __forceinline__ uint32_t ordered_bits(float v)
{
    if (v == 0.0f)
        v = 0.0f;                          // -0 == +0
    uint32_t u = __float_as_uint(v);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v)
{
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
        uint64_t o = __shfl_xor(v, d, 64);
        v = o > v ? o : v;
    }
    return v;
}

__global__ __launch_bounds__(kRouteWaves * 64) void route_kernel(int T, int E, int k,
                                                                 const float *__restrict__ logits,
                                                                 int32_t *__restrict__ ids,
                                                                 float *__restrict__ w)
{
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * kRouteWaves + (threadIdx.x >> 6);
    if (t >= T)
        return;
    const float *row = logits + (size_t)t * E;
    uint64_t key[kPerLane];
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) {
        int e = lane + 64 * i;
        key[i] = 0;
        if (e < E)
            key[i] = ((uint64_t)ordered_bits(row[e]) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)e);
    }
    float sel_v[kMaxTopK];
    int sel_e[kMaxTopK];
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
        if (j >= k)
            break;
        uint64_t best = 0;
#pragma unroll
        for (int i = 0; i < kPerLane; ++i)
            best = key[i] > best ? key[i] : best;
        best = wave_max_u64(best);
        const int e = (int)(0xFFFFFFFFu - (uint32_t)best);
        sel_e[j] = e;
        sel_v[j] = row[e];
        // the owner lane retires the winner
#pragma unroll
        for (int i = 0; i < kPerLane; ++i)
            if (lane + 64 * i == e)
                key[i] = 0;
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
        if (lane == j) {
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
    const int blocks = (T + kRouteWaves - 1) / kRouteWaves;
    hipLaunchKernelGGL(route_kernel, dim3(blocks), dim3(kRouteWaves * 64), 0, st, T,
                       sh.num_experts, sh.top_k, logits, ids, w);
    return hipGetLastError();
}

}  // namespace moe

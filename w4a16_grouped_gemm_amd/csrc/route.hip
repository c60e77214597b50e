// route.hip -- wavefront-level top-k routing with softmax renormalisation.
//
// 16 lanes per token (a DPP row) for E <= 256, a whole wave for larger E;
// lane q holds logits q, q+TL, ... . Each of k rounds takes the largest
// remaining logit (on an order-preserving integer image; -0 is folded to +0
// so equal logits tie exactly as IEEE equality says), then the lowest expert
// index holding it: the order (logit desc, index asc). The selection and the
// weights are in route_core.hpp.
#include "route_core.hpp"

namespace moe {

namespace {

constexpr int kRouteWaves = 4;

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
    int e;
    float wt;
    route_token<TL, PL>(logits + (size_t)t * E, E, k, q, e, wt);
    if (q < k) {
        ids[(size_t)t * k + q] = e;
        w[(size_t)t * k + q] = wt;
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

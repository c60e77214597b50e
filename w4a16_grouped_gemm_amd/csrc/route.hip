// route.hip -- wavefront-level top-k routing with softmax renormalisation.
//
// A whole wave per token up to 4096 tokens, else 16 lanes per token (a DPP
// row) for E <= 256 and a whole wave for larger E;
// lane q holds logits q, q+TL, ... . Each of k rounds takes the largest
// remaining logit (on an order-preserving integer image; -0 is folded to +0
// so equal logits tie exactly as IEEE equality says), then the lowest expert
// index holding it: the order (logit desc, index asc). The selection and the
// weights are in route_core.hpp.
#include "route_core.hpp"
#include "mx_quant.hpp"

namespace moe {

namespace {

constexpr int kRouteWaves = 4;
constexpr int kRouteQuantBatch = 4;                    // x blocks a thread loads before routing

// QX (the W4A4 layer): the launch also quantizes x [T][H] to MXFP4 (xq, xs),
// spread over all its threads; each thread's first blocks are loaded before
// its routing starts, so that their memory round trip overlaps it.
template <int TL, int PL, bool QX = false>
__global__ __launch_bounds__(kRouteWaves * 64) void route_kernel(int T, int E, int k,
                                                                 const float *__restrict__ logits,
                                                                 int32_t *__restrict__ ids,
                                                                 float *__restrict__ w,
                                                                 const uint16_t *__restrict__ x = nullptr, int H = 0,
                                                                 uint8_t *__restrict__ xq = nullptr,
                                                                 uint8_t *__restrict__ xs = nullptr)
{
    constexpr int TPW = 64 / TL;                       // tokens per wave
    const int lane = threadIdx.x & 63;
    const int q = lane % TL;                           // lane within the token
    const int t = (blockIdx.x * kRouteWaves + (threadIdx.x >> 6)) * TPW + lane / TL;
    const long long nblk = QX ? (long long)T * (H >> 5) : 0;
    const long long gt = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const long long gs = (long long)gridDim.x * blockDim.x;
    uint32_t xw[QX ? kRouteQuantBatch : 1][16];
    if constexpr (QX)
        mx_blocks_load<kRouteQuantBatch>(x, nblk, gt, gs, xw);
    if (t < T) {
        int e;
        float wt;
        route_token<TL, PL>(logits + (size_t)t * E, E, k, q, e, wt);
        if (q < k) {
            ids[(size_t)t * k + q] = e;
            w[(size_t)t * k + q] = wt;
        }
    }
    if constexpr (QX)
        mx_blocks_finish<kRouteQuantBatch>(xw, x, nblk, gt, gs, xq, xs);
}

}  // namespace

hipError_t launch_route(const moe_shape &sh, const float *logits, int32_t *ids, float *w,
                        hipStream_t st, const uint16_t *x, uint8_t *xq, uint8_t *xs)
{
    const int T = sh.num_tokens;
    const int E = sh.num_experts;
    const int k = sh.top_k;
    const int H = sh.hidden;
    const dim3 block(kRouteWaves * 64);
    auto grid = [&](int tl) { return dim3((T + kRouteWaves * (64 / tl) - 1) / (kRouteWaves * (64 / tl))); };
    if (x) {
        // the W4A4 layer: routing and the quantization of x in one launch
        // (a whole wave per token up to 4096 tokens, as below)
        if (T <= 4096 && E <= 256 && k <= 16) {
            if (E <= 64)
                hipLaunchKernelGGL((route_kernel<64, 1, true>), grid(64), block, 0, st, T, E, k, logits, ids, w, x, H, xq, xs);
            else if (E <= 128)
                hipLaunchKernelGGL((route_kernel<64, 2, true>), grid(64), block, 0, st, T, E, k, logits, ids, w, x, H, xq, xs);
            else
                hipLaunchKernelGGL((route_kernel<64, 4, true>), grid(64), block, 0, st, T, E, k, logits, ids, w, x, H, xq, xs);
            return hipGetLastError();
        }
        hipError_t e = launch_route(sh, logits, ids, w, st);
        if (e != hipSuccess)
            return e;
        return launch_mx_quantize(T, H, x, xq, xs, nullptr, st);
    }
    // A whole wave per token while that still leaves the GPU short of waves
    // (up to 4096 tokens: 1024 workgroups): the k selection rounds are the
    // serial part of routing, and 64 lanes of 2 logits (128 experts) take
    // about half the instructions per round of 16 lanes of 8. Same
    // selection and weights bit for bit (route_core.hpp).
    if (T <= 4096 && E <= 256 && k <= 16) {
        if (E <= 64)
            hipLaunchKernelGGL((route_kernel<64, 1>), grid(64), block, 0, st, T, E, k, logits, ids, w);
        else if (E <= 128)
            hipLaunchKernelGGL((route_kernel<64, 2>), grid(64), block, 0, st, T, E, k, logits, ids, w);
        else
            hipLaunchKernelGGL((route_kernel<64, 4>), grid(64), block, 0, st, T, E, k, logits, ids, w);
    } else if (E <= 64 && k <= 16)
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

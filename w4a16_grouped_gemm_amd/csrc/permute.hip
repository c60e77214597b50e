// permute.hip -- stable expert permutation: histogram, exclusive scan,
// token-stable scatter; plus the optional bf16 row gather.
//
// InfiniLM PR #500 report, section 2.2: bucket the routing ids into per-expert
// counts and a permutation, then gather rows by it. Here the bucketing runs on
// the device (no device-to-host copy, section 2.3's concern disappears) and is
// deterministic: atomics only count, and a slot's position is
//   offsets[e] + #{earlier tokens routed to e},
// computed from per-expert token bitmaps with popcounts. A token's k experts
// are distinct, so token order alone fixes every position.
//
// FlashInfer PR #7196 analysis, section 2 ("specialized BF16 permutation"):
// copy only the valid rows, with wide vectors; rows are 16-byte aligned here
// because H is a multiple of 128.
#include "common.hpp"
#include "mx_quant.hpp"
#include "route_core.hpp"

#include <mutex>

namespace moe {

namespace {

constexpr int kPermThreads = 1024;
constexpr int kMaskBytes = 32 * 1024;   // LDS budget for the token bitmaps
constexpr size_t kDynLdsMax = 144 * 1024; // dynamic LDS of one launch: bitmaps + staged ids (160 KiB per CU)

// One workgroup does the whole permutation: T*k <= 16M slots, E_loc <= 1024.
// IDS_IN_LDS: the routing ids are read from global memory once, coalesced,
// and every later pass reads LDS (each pass over global ids would cost a
// memory round trip per slot of a thread).
// ROUTE: the workgroup routes the tokens itself first (logits in, ids and
// weights written out as by moe_route, local ids kept in LDS), saving the
// separate routing launch and its round trip through memory. TL and PL are
// the routing shape (lanes per token, logits per lane).
// bases != NULL: the workgroup only scatters tokens [b*tpb, (b+1)*tpb) of the
// permutation (b = blockIdx.x); bases[b'*E + e] holds the slots of expert e
// in each range b' (permute_hist_kernel), from which every workgroup forms
// its own first rows (the parallel path for many tokens).
// QX (with ROUTE; the W4A4 layer): the workgroup also quantizes x [T][H]
// to MXFP4 (xq, xs); each thread's first blocks are loaded before routing.
template <bool IDS_IN_LDS, bool ROUTE = false, int TL = 16, int PL = 8, bool QX = false>
__global__ __launch_bounds__(kPermThreads) void permute_kernel(
    int T, int k, int begin, int E, const int32_t *__restrict__ ids, int32_t *__restrict__ counts,
    int32_t *__restrict__ offsets, int32_t *__restrict__ perm, int32_t *__restrict__ inv_perm,
    int chunk_tokens, const float *__restrict__ logits = nullptr, int E_g = 0,
    int32_t *__restrict__ ids_out = nullptr, float *__restrict__ w_out = nullptr, int num_shared = 0,
    const int32_t *__restrict__ bases = nullptr, int tpb = 0, const uint16_t *__restrict__ xsrc = nullptr,
    int H = 0, uint8_t *__restrict__ xq = nullptr, uint8_t *__restrict__ xs = nullptr)
{
    static_assert(!QX || ROUTE, "x is quantized by the routing workgroup");
    static_assert(!ROUTE || IDS_IN_LDS, "routing in the kernel keeps the ids in LDS");
    __shared__ int s_count[kMaxExperts];
    __shared__ int s_cursor[kMaxExperts];
    __shared__ int s_wave_tot[kPermThreads / 64];
    extern __shared__ uint32_t s_dyn[];
    const int tid = threadIdx.x;
    const int words = chunk_tokens >> 5;
    // token range of this workgroup: all tokens, or one range of the parallel path
    const int t_beg = bases ? (int)blockIdx.x * tpb : 0;
    const int t_end = bases ? min(T, t_beg + tpb) : T;
    const long long slot0 = (long long)t_beg * k;
    const long long S = (long long)(t_end - t_beg) * k;                 // slots of the range
    uint32_t *s_mask = s_dyn;                                           // [E][words]
    int *s_wprefix = reinterpret_cast<int *>(s_mask + (size_t)E * words);   // [E][words]
    int *s_ids = s_wprefix + (size_t)E * words;                         // [S] local expert or -1

    // All tokens in one bitmap chunk (the usual decode case): the per-expert
    // counts come from the bitmaps' popcounts, so the kernel needs four
    // barriers (ids, bitmaps, per-expert scan, wave totals) instead of a
    // histogram pass and a chunk loop.
    const bool one_chunk = !bases && T <= chunk_tokens && E <= kPermThreads;
    for (int e = tid; e < E; e += kPermThreads)
        s_count[e] = 0;
    if (one_chunk)
        for (int i = tid; i < E * words; i += kPermThreads)
            s_mask[i] = 0u;
    constexpr int kQB = 2;                            // x blocks a thread loads before routing
    uint32_t xw[QX ? kQB : 1][16];
    const long long nblk = QX ? (long long)T * (H >> 5) : 0;
    if constexpr (QX)
        mx_blocks_load<kQB>(xsrc, nblk, tid, kPermThreads, xw);
    if (ROUTE) {
        // 64 / TL tokens per wave and pass; a token's TL lanes form whole DPP rows
        constexpr int TPWV = 64 / TL;
        const int lane = tid & 63, q = lane % TL;
        for (int t0 = (tid >> 6) * TPWV; t0 < T; t0 += (kPermThreads / 64) * TPWV) {
            const int t = t0 + lane / TL;
            if (t < T) {
                int eg;
                float wt;
                route_token<TL, PL>(logits + (size_t)t * E_g, E_g, k, q, eg, wt);
                if (q < k) {
                    ids_out[(size_t)t * k + q] = eg;
                    w_out[(size_t)t * k + q] = wt;
                    const int e = eg - begin;
                    s_ids[t * k + q] = (e >= 0 && e < E) ? e : -1;
                }
            }
        }
        if constexpr (QX)
            mx_blocks_finish<kQB>(xw, xsrc, nblk, tid, kPermThreads, xq, xs);
    } else if (IDS_IN_LDS) {
        // local expert index (or -1) of every slot; four loads per thread go
        // out before the first is used (clamped indices, no branch)
        for (int base = 0; base < (int)S; base += 4 * kPermThreads) {
            int v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u)
                v[u] = ids[slot0 + min(base + u * kPermThreads + tid, (int)S - 1)];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int i = base + u * kPermThreads + tid;
                const int e = v[u] - begin;
                if (i < (int)S)
                    s_ids[i] = (e >= 0 && e < E) ? e : -1;
            }
        }
    }
    __syncthreads();
    auto local_expert = [&](long long slot) -> int {      // slot: global index t*k + j
        if (IDS_IN_LDS)
            return s_ids[slot - slot0];
        const int e = ids[slot] - begin;
        return (e >= 0 && e < E) ? e : -1;
    };

    if (one_chunk) {
        // bitmaps: bit t of expert e's words <=> token t routed to local e
        for (int t = tid; t < T; t += kPermThreads) {
            int le[kMaxTopK];                 // all of the token's ids first
#pragma unroll
            for (int j = 0; j < kMaxTopK; ++j)
                le[j] = local_expert((long long)t * k + min(j, k - 1));
#pragma unroll
            for (int j = 0; j < kMaxTopK; ++j)
                if (j < k && le[j] >= 0)
                    atomicOr(&s_mask[le[j] * words + (t >> 5)], 1u << (t & 31));
        }
        __syncthreads();
        // per expert (thread e): prefix popcounts over its words, its count,
        // and the exclusive scan of the counts across the workgroup
        const int e = tid;
        int cnt = 0;
        if (e < E)
            for (int wd = 0; wd < words; ++wd) {
                s_wprefix[e * words + wd] = cnt;
                cnt += __popc(s_mask[e * words + wd]);
            }
        int wtot;
        const int ex = wave_exclusive_scan(cnt, wtot);
        if ((tid & 63) == 0)
            s_wave_tot[tid >> 6] = wtot;
        __syncthreads();
        int wbase = 0, R = 0;
        for (int w = 0; w < kPermThreads / 64; ++w) {
            const int t = s_wave_tot[w];
            wbase += (w < (tid >> 6)) ? t : 0;
            R += t;
        }
        if (e < E) {
            offsets[e] = wbase + ex;
            counts[e] = cnt;
            s_cursor[e] = wbase + ex;
        }
        if (tid == 0)
            offsets[E] = R;
        for (int sh = tid; sh < num_shared; sh += kPermThreads) {
            counts[E + sh] = T;
            offsets[E + 1 + sh] = R + (sh + 1) * T;
        }
        for (long long r = tid; r < (long long)num_shared * T; r += kPermThreads)
            perm[R + r] = (int32_t)((r % T) * k);
        __syncthreads();
        for (int t = tid; t < T; t += kPermThreads) {
            int le[kMaxTopK];
#pragma unroll
            for (int j = 0; j < kMaxTopK; ++j)
                le[j] = local_expert((long long)t * k + min(j, k - 1));
#pragma unroll
            for (int j = 0; j < kMaxTopK; ++j) {
                if (j >= k)
                    break;
                const long long slot = (long long)t * k + j;
                const int le_j = le[j];
                int32_t row = -1;
                if (le_j >= 0) {
                    const uint32_t m = s_mask[le_j * words + (t >> 5)];
                    row = s_cursor[le_j] + s_wprefix[le_j * words + (t >> 5)] + __popc(m & ((1u << (t & 31)) - 1u));
                    perm[row] = (int32_t)slot;
                }
                inv_perm[slot] = row;
            }
        }
        for (long long r = R + (long long)num_shared * T + tid; r < S + (long long)num_shared * T; r += kPermThreads)
            perm[r] = -1;
        return;
    }

    int R = 0;
    if (bases) {
        // bases[b][e]: expert e's slots in token range b. Thread e sums its
        // column (its total, and the ranges before this one), the block scans
        // the totals into offsets; range b's slots of expert e start at
        // offsets[e] + (slots of e in ranges < b). Range 0 also writes the
        // counts, offsets, shared segments and the -1 rows.
        const int B = gridDim.x, b = blockIdx.x;
        const int e = tid;                                // E <= kPermThreads
        const int ec = min(e, E - 1);                     // clamped: loads never sit under a branch
        int total = 0, before = 0;
        for (int b0 = 0; b0 < B; b0 += 8) {
            int v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                v[j] = bases[(size_t)min(b0 + j, B - 1) * E + ec];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int vj = (b0 + j < B) ? v[j] : 0;
                total += vj;
                before += (b0 + j < b) ? vj : 0;
            }
        }
        if (e >= E)
            total = before = 0;
        int wtot;
        const int ex = wave_exclusive_scan(total, wtot);
        if ((tid & 63) == 0)
            s_wave_tot[tid >> 6] = wtot;
        __syncthreads();
        int wbase = 0;
        for (int w = 0; w < kPermThreads / 64; ++w) {
            const int t = s_wave_tot[w];
            wbase += (w < (tid >> 6)) ? t : 0;
            R += t;
        }
        if (e < E)
            s_cursor[e] = wbase + ex + before;
        if (b == 0) {
            if (e < E) {
                counts[e] = total;
                offsets[e] = wbase + ex;
            }
            if (tid == 0)
                offsets[E] = R;
            for (int sh = tid; sh < num_shared; sh += kPermThreads) {
                counts[E + sh] = T;
                offsets[E + 1 + sh] = R + (sh + 1) * T;
            }
            const long long S_all = (long long)T * k;
            for (long long r = tid; r < (long long)num_shared * T; r += kPermThreads)
                perm[R + r] = (int32_t)((r % T) * k);
            for (long long r = R + (long long)num_shared * T + tid; r < S_all + (long long)num_shared * T;
                 r += kPermThreads)
                perm[r] = -1;
        }
        __syncthreads();
    } else {
    // 1. histogram of local slots
    for (long long i = tid; i < S; i += kPermThreads) {
        const int e = local_expert(i);
        if (e >= 0)
            atomicAdd(&s_count[e], 1);
    }
    __syncthreads();

    // 2. exclusive scan over experts (one element per thread per pass)
    int carry = 0;
    for (int base = 0; base < E; base += kPermThreads) {
        int e = base + tid;
        int v = e < E ? s_count[e] : 0;
        int wtot;
        int ex = wave_exclusive_scan(v, wtot);
        if ((tid & 63) == 0)
            s_wave_tot[tid >> 6] = wtot;
        __syncthreads();
        int wbase = 0, all = 0;
        for (int w = 0; w < kPermThreads / 64; ++w) {
            int t = s_wave_tot[w];
            if (w < (tid >> 6))
                wbase += t;
            all += t;
        }
        if (e < E) {
            int off = carry + wbase + ex;
            offsets[e] = off;
            counts[e] = v;
            s_cursor[e] = off;
        }
        carry += all;
        __syncthreads();
    }
    if (tid == 0)
        offsets[E] = carry;
    R = carry;
    // shared experts (layer path only): expert E + s holds every token, row
    // R + s*T + t, whose perm entry t*k makes the GEMM read token t
    for (int sh = tid; sh < num_shared; sh += kPermThreads) {
        counts[E + sh] = T;
        offsets[E + 1 + sh] = R + (sh + 1) * T;
    }
    for (long long r = tid; r < (long long)num_shared * T; r += kPermThreads)
        perm[R + r] = (int32_t)((r % T) * k);
    }

    // 3. stable scatter, chunk by chunk of tokens
    for (int t0 = t_beg; t0 < t_end; t0 += chunk_tokens) {
        for (int i = tid; i < E * words; i += kPermThreads)
            s_mask[i] = 0u;
        __syncthreads();
        const int nt = min(chunk_tokens, t_end - t0);
        for (int tl = tid; tl < nt; tl += kPermThreads) {
            const int t = t0 + tl;
            int le[kMaxTopK];                 // all of the token's ids first: one round trip
#pragma unroll
            for (int j = 0; j < kMaxTopK; ++j)
                le[j] = local_expert((long long)t * k + min(j, k - 1));
#pragma unroll
            for (int j = 0; j < kMaxTopK; ++j)
                le[j] = j < k ? le[j] : -1;
#pragma unroll
            for (int j = 0; j < kMaxTopK; ++j)
                if (le[j] >= 0)
                    atomicOr(&s_mask[le[j] * words + (tl >> 5)], 1u << (tl & 31));
        }
        __syncthreads();
        // per-expert prefix popcounts over the chunk's words
        for (int e = tid; e < E; e += kPermThreads) {
            int run = 0;
            for (int wd = 0; wd < words; ++wd) {
                s_wprefix[e * words + wd] = run;
                run += __popc(s_mask[e * words + wd]);
            }
        }
        __syncthreads();
        for (int tl = tid; tl < nt; tl += kPermThreads) {
            const int t = t0 + tl;
            int le[kMaxTopK];
#pragma unroll
            for (int j = 0; j < kMaxTopK; ++j)
                le[j] = local_expert((long long)t * k + min(j, k - 1));
#pragma unroll
            for (int j = 0; j < kMaxTopK; ++j)
                le[j] = j < k ? le[j] : -1;
#pragma unroll
            for (int j = 0; j < kMaxTopK; ++j) {
                if (j >= k)
                    break;
                const long long slot = (long long)t * k + j;
                const int e = le[j];
                int32_t row = -1;
                if (e >= 0) {
                    const uint32_t m = s_mask[e * words + (tl >> 5)];
                    const int rank = s_wprefix[e * words + (tl >> 5)] +
                                     __popc(m & ((1u << (tl & 31)) - 1u));
                    row = s_cursor[e] + rank;
                    perm[row] = (int32_t)slot;
                }
                inv_perm[slot] = row;
            }
        }
        __syncthreads();
        for (int e = tid; e < E; e += kPermThreads)
            s_cursor[e] += s_wprefix[e * words + words - 1] + __popc(s_mask[e * words + words - 1]);
        __syncthreads();
    }
    // rows past the routed and shared rows hold no slot
    if (!bases)
        for (long long r = R + (long long)num_shared * T + tid; r < S + (long long)num_shared * T; r += kPermThreads)
            perm[r] = -1;
}

// Parallel path, step 1: expert histogram of each workgroup's token range
// (tpb tokens) -> part[b][e].
__global__ __launch_bounds__(256) void permute_hist_kernel(int T, int k, int begin, int E, int tpb,
                                                           const int32_t *__restrict__ ids,
                                                           int32_t *__restrict__ part)
{
    __shared__ int s_cnt[kMaxExperts];
    const int tid = threadIdx.x;
    for (int e = tid; e < E; e += 256)
        s_cnt[e] = 0;
    __syncthreads();
    const long long s0 = (long long)blockIdx.x * tpb * k;
    const long long s1 = min((long long)T, (long long)(blockIdx.x + 1) * tpb) * k;
    for (long long i = s0 + tid; i < s1; i += 256) {
        const int e = ids[i] - begin;
        if (e >= 0 && e < E)
            atomicAdd(&s_cnt[e], 1);
    }
    __syncthreads();
    for (int e = tid; e < E; e += 256)
        part[(size_t)blockIdx.x * E + e] = s_cnt[e];
}

// x_perm[r] = x[perm[r] / k] for r < R; 16 bytes per thread.
__global__ __launch_bounds__(256) void gather_kernel(int H, int k, int E,
                                                     const uint16_t *__restrict__ x,
                                                     const int32_t *__restrict__ perm,
                                                     const int32_t *__restrict__ offsets,
                                                     uint16_t *__restrict__ x_perm, long long max_rows)
{
    const int R = offsets[E];
    const int vec_per_row = H >> 3;
    const long long total = (long long)R * vec_per_row;
    for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (long long)gridDim.x * blockDim.x) {
        const long long r = i / vec_per_row;
        const int v = (int)(i - r * vec_per_row);
        if (r >= max_rows)
            break;
        const int src = perm[r] / k;
        const u32x4 d = *reinterpret_cast<const u32x4 *>(x + (size_t)src * H + (size_t)v * 8);
        *reinterpret_cast<u32x4 *>(x_perm + (size_t)r * H + (size_t)v * 8) = d;
    }
}

}  // namespace

static int chunk_tokens_for(int E)
{
    // bitmaps + prefix words: 8 bytes per (expert, 32 tokens)
    int c = 1024;
    while (c > 32 && (size_t)E * (c / 32) * 8 > (size_t)kMaskBytes)
        c >>= 1;
    return c;
}

// Past this many tokens (the launch override's permute_parallel_min_tokens
// can change it) the permutation runs over nb token ranges in two launches
// (per-range histograms, then a scatter whose workgroups each scan the
// histograms for their own first rows) instead of one workgroup; at most 64
// ranges, so that scan reads few partial counts per expert.
static int parallel_ranges(const moe_shape &sh)
{
    const int ov = launch_override().permute_parallel_min_tokens;
    const int min_t = ov >= 0 ? ov : 384;
    const int T = sh.num_tokens;
    if (T <= min_t || T < 2)
        return 0;
    return min(64, (T + 127) / 128);
}

size_t permute_workspace_bytes(const moe_shape &sh)
{
    return (size_t)parallel_ranges(sh) * sh.num_local_experts * sizeof(int32_t);
}

template <typename K>
static void allow_dyn_lds(K kernel)
{
    (void)hipFuncSetAttribute(reinterpret_cast<const void *>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)kDynLdsMax);
}

hipError_t launch_permute(const moe_shape &sh, const int32_t *ids, int32_t *counts,
                          int32_t *offsets, int32_t *perm, int32_t *inv_perm, hipStream_t st, int num_shared,
                          int32_t *part)
{
    static std::once_flag once;
    std::call_once(once, [] {
        allow_dyn_lds(permute_kernel<true>);
        allow_dyn_lds(permute_kernel<false>);
    });
    const int E = sh.num_local_experts;
    const int T = sh.num_tokens;
    const int nb = parallel_ranges(sh);
    const int tpb = nb ? (T + nb - 1) / nb : T;        // tokens per workgroup
    int chunk = chunk_tokens_for(E);
    while (chunk > 32 && chunk / 2 >= tpb)              // no wider than the token count needs
        chunk >>= 1;
    const size_t lds = (size_t)E * (chunk / 32) * 8;
    const long long S = (long long)tpb * sh.top_k;
    const bool ids_in_lds = lds + (size_t)S * 4 <= kDynLdsMax;
    const size_t dyn = ids_in_lds ? lds + (size_t)S * 4 : lds;
    if (nb) {
        if (!part)
            return hipErrorInvalidValue;
        hipLaunchKernelGGL(permute_hist_kernel, dim3(nb), dim3(256), 0, st, T, sh.top_k, sh.expert_begin, E, tpb,
                           ids, part);
    }
    const dim3 grid(nb ? nb : 1);
    if (ids_in_lds)
        hipLaunchKernelGGL(permute_kernel<true>, grid, dim3(kPermThreads), dyn, st, T, sh.top_k, sh.expert_begin, E,
                           ids, counts, offsets, perm, inv_perm, chunk, nullptr, 0, nullptr, nullptr, num_shared,
                           nb ? part : nullptr, tpb);
    else
        hipLaunchKernelGGL(permute_kernel<false>, grid, dim3(kPermThreads), dyn, st, T, sh.top_k, sh.expert_begin,
                           E, ids, counts, offsets, perm, inv_perm, chunk, nullptr, 0, nullptr, nullptr, num_shared,
                           nb ? part : nullptr, tpb);
    return hipGetLastError();
}

bool route_permute_fusable(const moe_shape &sh)
{
    const int E = sh.num_local_experts;
    int chunk = chunk_tokens_for(E);
    while (chunk > 32 && chunk / 2 >= sh.num_tokens)
        chunk >>= 1;
    const size_t lds = (size_t)E * (chunk / 32) * 8 + (size_t)sh.num_tokens * sh.top_k * 4;
    // One workgroup routes every token: it pays while routing is one pass of
    // its 16 waves (4 tokens each) and at most two waves share a SIMD; past that the separate routing launch,
    // spread over many CUs, is faster. The launch override's route_fuse_max_tokens can change it.
    const int ov = launch_override().route_fuse_max_tokens;
    const int max_t = ov >= 0 ? ov : 32;
    return sh.num_experts <= 256 && sh.num_tokens <= max_t && lds <= kDynLdsMax;
}

hipError_t launch_route_permute(const moe_shape &sh, const float *logits, int32_t *ids, float *w,
                                int32_t *counts, int32_t *offsets, int32_t *perm, int32_t *inv_perm,
                                hipStream_t st, int num_shared, const uint16_t *x, uint8_t *xq, uint8_t *xs)
{
    const int E = sh.num_local_experts;
    int chunk = chunk_tokens_for(E);
    while (chunk > 32 && chunk / 2 >= sh.num_tokens)
        chunk >>= 1;
    const size_t dyn = (size_t)E * (chunk / 32) * 8 + (size_t)sh.num_tokens * sh.top_k * 4;
    auto launch = [&](auto kernel) {
        if (dyn > 64 * 1024)
            (void)hipFuncSetAttribute(reinterpret_cast<const void *>(kernel),
                                      hipFuncAttributeMaxDynamicSharedMemorySize, (int)kDynLdsMax);
        hipLaunchKernelGGL(kernel, dim3(1), dim3(kPermThreads), dyn, st, sh.num_tokens, sh.top_k,
                           sh.expert_begin, E, nullptr, counts, offsets, perm, inv_perm, chunk, logits,
                           sh.num_experts, ids, w, num_shared, nullptr, 0, x, sh.hidden, xq, xs);
    };
    if (x) {
        if (sh.num_experts <= 64)
            launch(permute_kernel<true, true, 16, 4, true>);
        else if (sh.num_experts <= 128)
            launch(permute_kernel<true, true, 16, 8, true>);
        else
            launch(permute_kernel<true, true, 16, 16, true>);
    } else if (sh.num_experts <= 64)
        launch(permute_kernel<true, true, 16, 4>);
    else if (sh.num_experts <= 128)
        launch(permute_kernel<true, true, 16, 8>);
    else
        launch(permute_kernel<true, true, 16, 16>);
    return hipGetLastError();
}

hipError_t launch_gather(const moe_shape &sh, const uint16_t *x, const int32_t *perm,
                         const int32_t *offsets, uint16_t *x_perm, hipStream_t st)
{
    const long long rows = (long long)sh.num_tokens * sh.top_k;
    const long long total = rows * (sh.hidden / 8);
    long long blocks = (total + 255) / 256;
    const long long cap = (long long)device_cu_count() * 16;
    if (blocks > cap)
        blocks = cap;
    if (blocks < 1)
        blocks = 1;
    hipLaunchKernelGGL(gather_kernel, dim3((unsigned)blocks), dim3(256), 0, st, sh.hidden,
                       sh.top_k, sh.num_local_experts, x, perm, offsets, x_perm, rows);
    return hipGetLastError();
}

}  // namespace moe

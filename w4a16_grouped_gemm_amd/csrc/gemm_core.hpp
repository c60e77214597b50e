// gemm_core.hpp -- device building blocks shared by the grouped-GEMM kernels
// (gemm_w4a16.hip) and the small-batch layer kernels (decode.hip): buffer
// loads, the int4 unpack, the MFMA step, and the split-K tile body. The
// split-K body is one function used by every kernel that computes a tile
// that way, so they produce the same bits for the same tile.
//
// Method (pages): GC-MoE abstract (4-bit weights decoded in registers and fed
// straight to the matrix unit); Cloudflare "Unweight" post, section on the
// reconstructive matmul (weights rebuilt on chip, never written back).
#pragma once

#include "common.hpp"

namespace moe {

constexpr uint32_t kNeg136 = 0xC308C308u;  // bf16 pair (-136, -136)
constexpr uint32_t kOutOfRange = 0x80000000u;   // buffer offset past every descriptor
constexpr int kXcds = 8;                         // MI355X: 8 XCDs of 32 CUs, one L2 each

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// Cache policy of the weight-code stream. NT: non-temporal (the nt bit of
// the buffer instruction), for launches where each expert's codes are read
// about once (at most one chunk per expert): the streaming policy keeps
// them from evicting the activation rows, which the other blocks of a chunk
// read again from L2. Measured on MI355X (Qwen3-30B-A3B decode, 16-256
// tokens; the EP shard): both grouped GEMMs 6-9% faster. Where several
// chunks of an expert re-read its codes (prefill, a dense GEMM of many rows)
// the default policy keeps them in L2 for the next chunk (nt: 3-14% slower).
template <bool NT>
__device__ __forceinline__ u32x4 bload16_codes(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, NT ? 2 : 0));
}

// Raw bf16 bits of a scale; converted where it is used, so that the load can
// stay in flight until then (a conversion next to the load would wait for it).
__device__ __forceinline__ uint32_t bload_scale(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    return __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
}

// Nibbles j and j+4 -> bf16 pair j (128 + (q+8)): K order (0,4,1,5,..) for
// plain codes, column order for tiled ones.
__device__ __forceinline__ bf16x8 unpack8(uint32_t w)
{
    u32x4 o;
    o.x = (w & 0x000F000Fu) ^ 0x43084308u;
    o.y = ((w >> 4) & 0x000F000Fu) ^ 0x43084308u;
    o.z = ((w >> 8) & 0x000F000Fu) ^ 0x43084308u;
    o.w = ((w >> 12) & 0x000F000Fu) ^ 0x43084308u;
    return __builtin_bit_cast(bf16x8, o);
}

// Eight consecutive bf16 activations -> the (0,4,1,5,2,6,3,7) order of
// plain codes.
__device__ __forceinline__ u32x4 permute_act(u32x4 d)
{
    u32x4 o;
    o.x = __builtin_amdgcn_perm(d.z, d.x, 0x05040100u);
    o.y = __builtin_amdgcn_perm(d.z, d.x, 0x07060302u);
    o.z = __builtin_amdgcn_perm(d.w, d.y, 0x05040100u);
    o.w = __builtin_amdgcn_perm(d.w, d.y, 0x07060302u);
    return o;
}

__device__ __forceinline__ floatx4 mfma(u32x4 a, bf16x8 b, floatx4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), b, c, 0, 0, 0);
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + expf(-g)); }

// silu for a value that is rounded to bf16 next: hardware exp2 and reciprocal
// (errors of a few fp32 ulp, far below the bf16 rounding step).
__device__ __forceinline__ float silu_fast(float g)
{
    return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * g));
}

// Value of lane (l ^ 8) within each 16-lane row (DPP row rotate by 8).
__device__ __forceinline__ float row_swap8(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false));
}

__device__ __forceinline__ bf16x8 neg136_operand()
{
    const u32x4 v = {kNeg136, kNeg136, kNeg136, kNeg136};
    return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Group range [g0, g1) of wave `wave` when NW waves split G groups.
__device__ __forceinline__ void splitk_groups(int wave, int G, int NW, int &g0, int &g1)
{
    g0 = wave * G / NW;
    g1 = (wave + 1) * G / NW;
}

// One 128-wide group of a 16-row weight tile: the chain of the -136 * sum(x)
// correction MFMAs followed by the four code MFMAs (activation fragments a,
// already in the codes' K order), times the group's scale, added to tot.
__device__ __forceinline__ void splitk_group(const u32x4 (&a)[4], u32x4 wv, uint32_t sc, floatx4 &tot)
{
    const bf16x8 neg136 = neg136_operand();
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i)
        acc = mfma(a[i], neg136, acc);
    acc = mfma(a[0], unpack8(wv.x), acc);
    acc = mfma(a[1], unpack8(wv.y), acc);
    acc = mfma(a[2], unpack8(wv.z), acc);
    acc = mfma(a[3], unpack8(wv.w), acc);
    const float scale = bf16_to_f32(sc);
    tot.x = __builtin_fmaf(scale, acc.x, tot.x);
    tot.y = __builtin_fmaf(scale, acc.y, tot.y);
    tot.z = __builtin_fmaf(scale, acc.z, tot.z);
    tot.w = __builtin_fmaf(scale, acc.w, tot.w);
}

// One wave's share of a 16-row weight tile over groups [g0, g1): the sum over
// those groups, in ascending order, of scale_g * (chain of group g), the
// chain being the -136 * sum(x) correction MFMAs followed by the four code
// MFMAs (the per-group contraction is exact for integer activations).
// Loads go out GB groups at a time, all before the first is used; groups
// past g1 are not loaded. Activation fragments come from `ra` at voff_x
// (+16 per MFMA step, +256 per group; an out-of-range voff_x gives zeros).
template <int GB>
__device__ __forceinline__ floatx4 splitk_wave_sum(__amdgpu_buffer_rsrc_t rw, uint32_t voff_w, uint32_t gstride,
                                                   __amdgpu_buffer_rsrc_t rs, uint32_t voff_s,
                                                   __amdgpu_buffer_rsrc_t ra, uint32_t voff_x, int g0, int g1,
                                                   bool w_tiled)
{
    floatx4 tot = {0.f, 0.f, 0.f, 0.f};
    for (int gb = g0; gb < g1; gb += GB) {
        u32x4 wv[GB];
        uint32_t sc[GB];
        u32x4 xa[GB][4];
#pragma unroll
        for (int j = 0; j < GB; ++j) {
            if (gb + j < g1) {
                const uint32_t g = gb + j;
                wv[j] = bload16_codes<true>(rw, voff_w, g * gstride);
                sc[j] = bload_scale(rs, voff_s, g * 2);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    xa[j][i] = bload16(ra, voff_x + i * 16, g * kGroup * 2);
            }
        }
#pragma unroll
        for (int j = 0; j < GB; ++j) {
            if (gb + j >= g1)
                break;
            // a branch on the layout, not a select: with tiled codes the
            // fragments are used as loaded and no permutation is formed
            if (w_tiled) {
                splitk_group(xa[j], wv[j], sc[j], tot);
            } else {
                u32x4 a[4];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    a[i] = permute_act(xa[j][i]);
                splitk_group(a, wv[j], sc[j], tot);
            }
        }
    }
    return tot;
}

// Sum of the NW waves' shares in wave order (s_red[0] + s_red[1] + ...),
// valid in wave 0. Block-wide (two barriers): every wave must call it.
template <int NW>
__device__ __forceinline__ floatx4 splitk_reduce(floatx4 tot, floatx4 (*s_red)[64], int wave, int lane)
{
    s_red[wave][lane] = tot;
    __syncthreads();
    floatx4 sum = s_red[0][lane];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
        const floatx4 v = s_red[w][lane];
        sum.x += v.x;
        sum.y += v.y;
        sum.z += v.z;
        sum.w += v.w;
    }
    __syncthreads();
    return sum;
}

// Row offset of expert e: offsets[e], or for a dense GEMM (offsets NULL,
// one expert) 0 and dense_rows.
__device__ __forceinline__ int expert_offset(const int32_t *offsets, int dense_rows, int e)
{
    return offsets ? offsets[e] : (e == 0 ? 0 : dense_rows);
}

// Chunk prefix over experts: s_prefix[e] = chunks of experts < e (chunk =
// up to CS rows of one expert), s_prefix[E] = total. Block-wide.
// When s_off is given it receives offsets[0..E] as well.
template <int NT>
__device__ void build_chunk_prefix(const int32_t *offsets, int dense_rows, int E, int CS, int *s_prefix,
                                   int *s_wtot, int *s_off = nullptr)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int carry = 0;
    for (int base = 0; base < E; base += NT) {
        const int e = base + tid;
        int v = 0;
        if (e < E) {
            const int o0 = expert_offset(offsets, dense_rows, e), o1 = expert_offset(offsets, dense_rows, e + 1);
            if (s_off) {
                s_off[e] = o0;
                if (e == E - 1)
                    s_off[E] = o1;
            }
            const int cnt = o1 - o0;
            v = (cnt + CS - 1) / CS;
        }
        int wt;
        const int ex = wave_exclusive_scan(v, wt);
        if (lane == 0)
            s_wtot[wave] = wt;
        __syncthreads();
        int wbase = 0, all = 0;
#pragma unroll
        for (int w = 0; w < NT / 64; ++w) {
            wbase += (w < wave) ? s_wtot[w] : 0;
            all += s_wtot[w];
        }
        if (e < E)
            s_prefix[e] = carry + wbase + ex;
        carry += all;
        __syncthreads();
    }
    if (tid == 0)
        s_prefix[E] = carry;
    __syncthreads();
}

// Expert owning chunk `chunk`: the last e with s_prefix[e] <= chunk.
__device__ __forceinline__ int chunk_expert(const int *s_prefix, int E, int chunk)
{
    int lo = 0, hi = E - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_prefix[mid] <= chunk)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

// The same expert found by the whole wave at once (every lane active, chunk
// uniform): the prefix is non-decreasing, so the experts e >= 1 with
// s_prefix[e] <= chunk are exactly 1 .. answer, and the lanes count them in
// one pass of independent LDS reads per 64 experts instead of a chain of
// log2(E) dependent ones.
__device__ __forceinline__ int chunk_expert_wave(const int *s_prefix, int E, int chunk, int lane)
{
    int n = 0;
#pragma unroll 2
    for (int e0 = 1; e0 < E; e0 += 64) {
        const int e = e0 + lane;
        const int pv = s_prefix[e < E ? e : E];      // entry E exists: no load under a branch
        n += __popcll(__ballot((e < E) & (pv <= chunk)));
    }
    return n;
}

// ---------------------------------------------------------------------------
// SRC_IDS: the layer's stable expert permutation (moe_permute's result) built
// by every workgroup in LDS from the routing ids, so that the gate/up GEMM
// needs no permutation launch before it (InfiniLM PR #500 report, section
// 2.2: counts, offsets and a permutation from the routing ids). A token's k
// experts are distinct, so the rows of local expert e are its slots in token
// order: row(slot s of token t) = offsets[e] + #{tokens t' < t routed to e},
// counted from per-expert token bitmaps. Fills s_off / s_prefix as
// build_chunk_prefix does from `offsets`, and s_row[r] = slot of row r;
// workgroup 0 also stores counts, offsets, perm and inv_perm (-1 for a slot
// whose expert is not local). The bitmaps and word prefixes are scratch
// (dead after the last barrier). Needs E <= NT and T * k <= kIdsPerThread * NT.
// Used by the W4A16 streaming kernel and the W4A4 (MXFP4) LDS kernel.
// ---------------------------------------------------------------------------
constexpr int kIdsPerThread = 16;                 // slots per thread: T * k <= 16 * 256

struct IdsTables {
    const int32_t *ids;          // [T*k] global expert ids (the routing result)
    int T, k, begin, E;          // tokens, slots per token, global id of local expert 0, local experts
    int32_t *cnt_out, *off_out, *perm_out, *inv_out;   // stored by workgroup 0
    int nsh;                     // shared experts after the E routed ones (T rows each), as moe_permute appends them
};

template <int NT>
__device__ void build_from_ids(const IdsTables &p, int CS, uint32_t *s_bits, int *s_wpre, uint16_t *s_row,
                               int *s_prefix, int *s_off, int *s_wtot)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int E = p.E, k = p.k;
    const int S = p.T * k, words = (p.T + 31) >> 5;
    const bool store = blockIdx.x == 0;
    // every id load of the thread goes out before the first is used (one
    // memory round trip; slots past S read out of range, as zeros)
    const __amdgpu_buffer_rsrc_t rids = make_rsrc(p.ids, (uint32_t)S * 4u);
    int le[kIdsPerThread], tk[kIdsPerThread];          // local expert (-1: none) and token of each slot
#pragma unroll
    for (int j = 0; j < kIdsPerThread; ++j)
        le[j] = (int)__builtin_amdgcn_raw_buffer_load_b32(rids, (uint32_t)(tid + j * NT) * 4u, 0, 0);
    for (int i = tid; i < E * words; i += NT)
        s_bits[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kIdsPerThread; ++j) {
        const int s = tid + j * NT;
        const int e = le[j] - p.begin;
        le[j] = (s < S && e >= 0 && e < E) ? e : -1;
        tk[j] = s / k;
        if (le[j] >= 0)
            atomicOr(&s_bits[le[j] * words + (tk[j] >> 5)], 1u << (tk[j] & 31));
    }
    __syncthreads();
    // thread e: its row count and word prefixes, then one scan over the
    // experts of (rows, chunks of CS rows)
    // (experts E .. E + nsh - 1: the shared experts, every token once)
    const int Et = E + p.nsh;
    int cnt = 0, ch = 0;
    if (tid < E) {
        for (int w = 0; w < words; ++w) {
            s_wpre[tid * words + w] = cnt;
            cnt += __popc(s_bits[tid * words + w]);
        }
    } else if (tid < Et) {
        cnt = p.T;
    }
    ch = (cnt + CS - 1) / CS;
    int tc, tch;
    const int xc = wave_exclusive_scan(cnt, tc);
    const int xch = wave_exclusive_scan(ch, tch);
    if (lane == 0) {
        s_wtot[wave] = tc;
        s_wtot[NT / 64 + wave] = tch;
    }
    __syncthreads();
    int bc = 0, bch = 0, ac = 0, ach = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
        bc += w < wave ? s_wtot[w] : 0;
        bch += w < wave ? s_wtot[NT / 64 + w] : 0;
        ac += s_wtot[w];
        ach += s_wtot[NT / 64 + w];
    }
    if (tid < Et) {
        s_off[tid] = bc + xc;
        s_prefix[tid] = bch + xch;
        if (store) {
            p.cnt_out[tid] = cnt;
            p.off_out[tid] = bc + xc;
        }
    }
    if (tid == 0) {
        s_off[Et] = ac;
        s_prefix[Et] = ach;
        if (store)
            p.off_out[Et] = ac;
    }
    __syncthreads();
    // shared rows: row R + s T + t reads token t (slot t k, as moe_permute writes it)
    if (p.nsh > 0) {
        const int R = s_off[E];
        for (int r = tid; r < p.nsh * p.T; r += NT) {
            const int t = r % p.T;
            s_row[R + r] = (uint16_t)(t * k);
            if (store)
                p.perm_out[R + r] = t * k;
        }
    }
    // the row of every slot first (LDS reads only, all independent), then the stores
    int row[kIdsPerThread];
#pragma unroll
    for (int j = 0; j < kIdsPerThread; ++j) {
        const int e = le[j] >= 0 ? le[j] : 0, w = le[j] >= 0 ? tk[j] >> 5 : 0;
        const uint32_t below = s_bits[e * words + w] & ((1u << (tk[j] & 31)) - 1u);
        row[j] = s_off[e] + s_wpre[e * words + w] + __popc(below);
    }
#pragma unroll
    for (int j = 0; j < kIdsPerThread; ++j) {
        const int s = tid + j * NT;
        if (le[j] >= 0) {
            s_row[row[j]] = (uint16_t)s;
            if (store)
                p.perm_out[row[j]] = s;
        }
        if (store && s < S)
            p.inv_out[s] = le[j] >= 0 ? row[j] : -1;
    }
    __syncthreads();
}

// SRC_IDS scratch inside the activation buffers (bitmaps, word prefixes).
constexpr size_t ids_scratch_bytes(int E, int T)
{
    return (size_t)E * ((T + 31) / 32) * 8;
}

// ---- the layer's small-batch path: slot tables ------------------------------
// With at most 16 tokens every expert holds at most 16 routed rows, so a
// workgroup that knows each slot's local expert (s_loc[s], -1 when not local;
// slot s = t * k + j) can list an expert's rows itself: the "leader" of an
// expert is its first slot; its rows are its slots in slot order.

// Slot of row r of an expert whose slots are the set bits of (m0, m1): the
// r-th set bit, or -1 past the last.
__device__ __forceinline__ int nth_slot(uint64_t m0, uint64_t m1, int r)
{
    const int c0 = __popcll(m0);
    uint64_t m = r < c0 ? m0 : m1;
    int rr = r < c0 ? r : r - c0;
    if (rr >= __popcll(m))
        return -1;
    for (int i = 0; i < rr; ++i)
        m &= m - 1;
    return (r < c0 ? 0 : 64) + __builtin_ctzll(m);
}

// Shared slot bookkeeping of the two expert-major kernels, after s_loc[s]
// (local expert of slot s, or -1) is in LDS: s_first[e] = first slot of
// expert e, then the leaders in slot order in s_lead. Block-wide.
template <int NT>
__device__ void build_leaders(int S, int E_loc, const int *s_loc, int *s_first, int *s_lead, int *s_nlead)
{
    const int tid = threadIdx.x, lane = tid & 63;
    for (int s = tid; s < S; s += NT)
        if (s_loc[s] >= 0)
            atomicMin(&s_first[s_loc[s]], s);
    __syncthreads();
    if (tid < 64) {
        int base = 0;
        for (int s0 = 0; s0 < S; s0 += 64) {
            const int s = s0 + lane;
            const bool lead = s < S && s_loc[s] >= 0 && s_first[s_loc[s]] == s;
            const uint64_t m = __ballot(lead);
            if (lead)
                s_lead[base + __popcll(m & ((1ull << lane) - 1ull))] = s;
            base += __popcll(m);
        }
        if (lane == 0)
            *s_nlead = base;
    }
    __syncthreads();
}

// K-group count -> waves of a split-K tile (at least 2 groups per wave from
// 4 groups on; 8 waves once there are 24 groups or more).
constexpr int splitk_waves(int G) { return G >= 24 ? 8 : G >= 8 ? 4 : G >= 4 ? 2 : 1; }

}  // namespace moe

// gemm_w4a16.hip -- grouped GEMM over expert slabs, int4 group-scaled weights
// x bf16 activations, fp32 accumulation on gfx950 MFMA.
//
// Method (pages): InfiniLM PR #500 report, section 2.2 (one grouped GEMM
// covers every expert slab given the group sizes; gate/up, SwiGLU, down);
// FlashInfer PR #7196 analysis, section 2 (the MMA N extent follows the
// routed-token count at run time and inactive subtiles are skipped; the
// activations sit in operand B of an operand-swapped MMA; valid rows only);
// GC-MoE abstract (4-bit weights decoded in registers and fed straight to the
// matrix unit; decode is bound by weight traffic); Cloudflare "Unweight" post,
// section on the reconstructive matmul (weights are rebuilt on chip and never
// written back to HBM).
//
// gfx950 design (ours):
//  * MFMA v_mfma_f32_16x16x32_bf16. Operand A = 16 routed tokens of one
//    expert (a 16-token subtile of the expert's rows), operand B = 16 weight
//    rows. Lane l supplies token / weight row l%16 and one 8-element K slice
//    chosen by l/16; the result lane holds 4 tokens x 1 weight row, so a lane
//    needs one scale per 128-wide group: the scale of its own row.
//  * Weights stream HBM -> VGPR through buffer loads (SGPR descriptor per
//    expert, 32-bit lane offsets, group offsets folded into the instruction),
//    16 bytes per lane per group and 16-row tile (= 32 int4 codes of one row).
//    A lane's 32 codes feed 4 MFMAs.
//  * Unpack: ((w >> 4j) & 0x000F000F) ^ 0x43084308 turns nibbles j and j+4
//    into the bf16 values 128 + (q + 8) -- exact -- in one v_bitop3_b32 (plus
//    a shift shared by the 8 codes of the dword). With plain codes the K
//    order inside each dword comes out as (0,4,1,5,2,6,3,7) and activation
//    fragments are permuted the same way when they are staged (a common K
//    permutation leaves the dot product unchanged; the matrix unit's result
//    does not depend on the order of a lane's 8 K values). The tiled layout
//    stores each word's codes pre-shuffled so they unpack in column order,
//    and activations are then used as they lie in memory.
//  * The +136 offset is removed inside the matrix unit: per 16-token subtile
//    and group a chain of MFMAs against a constant -136 operand gives
//    -136 * sum(x); every weight tile's chain starts from it, so the chain
//    ends at sum(x * q) (exact for integer-valued activations). The row's
//    fp32 scale is applied once per group: total += s * chain. Codes are
//    never rounded.
//  * gemm_stream_kernel (the common case): a workgroup owns a block of
//    4 waves x TPW tiles x 16 weight rows over the full K for one chunk of up
//    to 16*NSUB rows of one expert. The chunk's activations are staged per
//    K-segment of KSEG groups into LDS (double buffered, one barrier per
//    segment), already in MFMA fragment order, and shared by the four waves,
//    each reusing them across its TPW tiles; weights are prefetched one
//    group ahead in registers. Tokens past the chunk are loaded as zeros by
//    the buffer unit's range check, so no lane branches on them.
//  * gemm_splitk_kernel (about one routed row per active expert, e.g. one
//    decode token): one 16-row tile per workgroup, K split over the waves,
//    partial sums reduced through LDS in wave order (deterministic). It keeps
//    many more workgroups in flight when only a few experts are active.
//  * Work items = (expert chunk, weight-row block). Every workgroup of a
//    persistent grid derives the item list on the device from `offsets`, so
//    the grid never depends on the counts and the host never synchronises.
//    Subtiles past the chunk's valid rows are skipped (runtime N); rows past
//    the last valid token are neither read nor written.
#include "gemm_core.hpp"
#include "route_core.hpp"

#include <map>
#include <type_traits>
#include <mutex>
#include <utility>

namespace moe {

namespace {

struct GemmArgs {
    const uint16_t *a;
    const int32_t *a_row_index;
    const int32_t *offsets;     // [E+1] on the device; NULL for one dense expert of dense_rows rows
    int dense_rows;
    const uint8_t *wq;
    const uint16_t *s;
    const uint8_t *wq_sh;        // experts e >= e_routed: shared experts, weights at index e - e_routed
    const uint16_t *s_sh;
    int e_routed;
    void *c;
    const int32_t *c_row_index;  // output row r goes to row c_row_index[r] (NULL: row r)
    uint32_t c_row_bytes;        // bytes of c_row_index (0 when NULL)
    uint32_t a_row_bytes;        // bytes of a_row_index (0 when NULL)
    uint32_t c_bytes;            // bytes of c the tile kernel's buffer stores reach (< 2^31)
    uint32_t a_bytes;  // bytes of `a` reachable through the buffer descriptor (< 2^31)
    int top_k;
    int num_experts;
    int K;
    int N;          // weight rows per expert
    int ldc;        // output row stride (elements)
    int half;       // SwiGLU: row offset of the up projection (= I)
    int c_f32;
    int w_tiled;    // codes in the tiled layout: tile t, group g at ((t/8)*G*8 + t%8)*1 KiB + g*8 KiB
    // the layer's small-batch item sources (gemm_stream_kernel with SRC != 0):
    // each expert's rows are its slots, listed from a slot table in LDS
    const float *logits;  // SRC_ROUTE: router logits [T][E_g]
    int T, E_g, begin;    // tokens, logit columns, global id of local expert 0
    int32_t *ids;         // per slot t*k+j: global expert id (SRC_ROUTE writes, SRC_SLOTS reads)
    float *wts;           // SRC_ROUTE writes the routing weights
    int32_t *pres;        // per slot: the slot index if its expert is local, else -1
    // SRC_IDS: the permutation's tables, stored by workgroup 0 as moe_permute would
    int32_t *cnt_out, *off_out, *perm_out, *inv_out;
};

// Item sources of the streaming kernel: the chunk prefix over `offsets`
// (the grouped GEMM), the small-batch layer's slot table, built by routing
// inside the kernel (gate/up) or read from the stored table (down), or the
// layer's permutation built from the routing ids inside the kernel (gate/up).
enum { SRC_OFFSETS = 0, SRC_ROUTE = 1, SRC_SLOTS = 2, SRC_IDS = 3 };

// Lane offset of a tile's codes and the byte step from one group to the next.
__device__ __forceinline__ uint32_t code_offset(const GemmArgs &p, int tile, uint32_t row, int G, uint32_t row_bytes,
                                                int lane)
{
    if (p.w_tiled)
        return (uint32_t)((tile >> 3) * G * 8 + (tile & 7)) * 1024u + (uint32_t)lane * 16u;
    return row * row_bytes + (uint32_t)(lane >> 4) * 16u;
}

__device__ __forceinline__ uint32_t group_stride(const GemmArgs &p) { return p.w_tiled ? 8192u : 64u; }


// Codes and scales of expert e: the routed arrays, or past e_routed the
// shared experts' arrays (e is uniform: a scalar select, no branch).
__device__ __forceinline__ const uint8_t *expert_codes(const GemmArgs &p, int e, uint32_t bytes)
{
    return e < p.e_routed ? p.wq + (size_t)e * bytes : p.wq_sh + (size_t)(e - p.e_routed) * bytes;
}

__device__ __forceinline__ const uint16_t *expert_scales(const GemmArgs &p, int e, uint32_t n)
{
    return e < p.e_routed ? p.s + (size_t)e * n : p.s_sh + (size_t)(e - p.e_routed) * n;
}

// Weight row of lane n16 in 16-row tile `tile`: for SwiGLU rows 0..7 are gate
// rows of features 8*tile.., rows 8..15 the matching up rows.
template <int KIND>
__device__ __forceinline__ int tile_row(const GemmArgs &p, int tile, int n16)
{
    if (KIND == MOE_GEMM_W13_SWIGLU)
        return (n16 < 8) ? tile * 8 + n16 : p.half + tile * 8 + (n16 - 8);
    return tile * 16 + n16;
}

// Store one lane's 4 results (tokens 4*kq+i of the subtile, row n16 of tile).
// Output row of result row r: r itself, or c_row_index[r] (read here unless
// the caller preloaded it into pre[i] for rows mbase + i).
__device__ __forceinline__ int out_row(const GemmArgs &p, int r, const int *pre, int i)
{
    if (!p.c_row_index)
        return r;
    return pre ? pre[i] : p.c_row_index[r];
}

template <int KIND>
__device__ __forceinline__ void store_tile(const GemmArgs &p, floatx4 v, int tile, int row0, int mbase,
                                           int nvalid, int n16, const int *pre = nullptr)
{
    float r[4] = {v.x, v.y, v.z, v.w};
    if (KIND == MOE_GEMM_W13_SWIGLU) {
        float u[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            u[i] = __shfl_xor(r[i], 8, 64);            // partner lane holds the up row
        if (n16 < 8) {
            uint16_t *c = static_cast<uint16_t *>(p.c);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = mbase + i;
                if (m < nvalid)
                    c[(size_t)out_row(p, row0 + m, pre, i) * p.ldc + tile * 8 + n16] =
                        (uint16_t)f32_to_bf16_rne(silu(r[i]) * u[i]);
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = mbase + i;
            if (m < nvalid) {
                const size_t off = (size_t)out_row(p, row0 + m, pre, i) * p.ldc + tile * 16 + n16;
                if (p.c_f32)
                    static_cast<float *>(p.c)[off] = r[i];
                else
                    static_cast<uint16_t *>(p.c)[off] = (uint16_t)f32_to_bf16_rne(r[i]);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// gemm_stream_kernel
//
// No load sits under a branch: tiles past N never occur (the host launches
// this kernel only when 4*TPW tiles divide N), tokens past the chunk, groups
// past K and the segment after the last are all loaded through out-of-range
// buffer offsets (zeros, no memory traffic). The waitcnt insertion then sees
// one straight sequence of loads, so each wait names exactly the load it
// needs and the weight ring stays in flight across groups.
// ---------------------------------------------------------------------------
template <int NSUB, int KSEG>
constexpr size_t stream_act_bytes()
{
    return sizeof(u32x4) * 2 * KSEG * NSUB * 4 * 64;
}

// LDS slot of MFMA step `step`, lane `lane` inside one 64-slot row: the low
// four lane bits are XORed with (4*step + lane/16) so that the staging
// writes (16 lanes of one token, all steps) and the MFMA reads (16 lanes of
// one step) both hit 16 distinct 16-byte bank groups.
__device__ __forceinline__ int act_slot(int step, int lane)
{
    return lane ^ ((4 * step + (lane >> 4)) & 15);
}

template <int KIND, int TPW, int NSUB, int KSEG, int RING, bool NT, int SRC = SRC_OFFSETS, int PL = 8>
__global__ __launch_bounds__(256) void gemm_stream_kernel(GemmArgs p)
{
    static_assert(SRC == SRC_OFFSETS || SRC == SRC_IDS || NSUB == 1, "small-batch items hold at most 16 rows");
    constexpr bool CHUNKED = SRC == SRC_OFFSETS || SRC == SRC_IDS;   // items from the chunk prefix
    static_assert((2 * KSEG) % RING == 0, "the weight ring slot of group g is g % RING, static per segment parity");
    static_assert(KSEG == 1 || KSEG % 2 == 0, "scales are loaded as dwords of two groups");
    constexpr int SD = (KSEG + 1) / 2;                 // scale dwords per tile and segment
    constexpr int CS = 16 * NSUB;
    constexpr int BT = 4 * TPW;                         // tiles per block
    extern __shared__ __align__(16) unsigned char s_dyn[];
    // [buf][group][subtile][step][slot] activation fragments, then the chunk
    // prefix, the expert offsets and the scan scratch
    auto s_act = reinterpret_cast<u32x4(*)[KSEG][NSUB][4][64]>(s_dyn);
    const int E = p.num_experts;
    int *s_prefix = reinterpret_cast<int *>(s_dyn + stream_act_bytes<NSUB, KSEG>());
    int *s_off = s_prefix + (E + 1);
    int *s_wtot = s_off + (E + 1);
    // small-batch slot tables (SRC != 0), in the same region
    int *s_loc = s_prefix;
    int *s_lead = s_loc + kDecMaxSlots;
    int *s_nlead = s_lead + kDecMaxSlots;
    int *s_first = s_nlead + 4;
    // SRC_IDS: slot of each permuted row, after the scan scratch (2 x 4 ints)
    uint16_t *s_row = reinterpret_cast<uint16_t *>(s_wtot + 8);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int n16 = lane & 15;
    const int kq = lane >> 4;
    const int ntiles = p.N >> 4;
    const int nblocks = ntiles / BT;
    const int S_slots = p.T * p.top_k;
    int total_items;
    if constexpr (SRC == SRC_OFFSETS) {
        build_chunk_prefix<256>(p.offsets, p.dense_rows, E, CS, s_prefix, s_wtot, s_off);
        total_items = s_prefix[E] * nblocks;
    } else if constexpr (SRC == SRC_IDS) {
        uint32_t *s_bits = reinterpret_cast<uint32_t *>(s_dyn);
        const int words = (p.T + 31) >> 5;
        int *s_wpre = reinterpret_cast<int *>(s_bits + E * words);
        // (the shared experts, if any, are the last E - e_routed)
        const IdsTables it{p.ids,      p.T,        p.top_k,     p.begin,   p.e_routed,
                           p.cnt_out,  p.off_out,  p.perm_out,  p.inv_out, E - p.e_routed};
        build_from_ids<256>(it, CS, s_bits, s_wpre, s_row, s_prefix, s_off, s_wtot);
        total_items = s_prefix[E] * nblocks;
    } else {
        for (int e = tid; e < E; e += 256)
            s_first[e] = kDecMaxSlots;
        if constexpr (SRC == SRC_ROUTE) {
            // every workgroup routes all tokens: one DPP row of 16 lanes per token
            for (int t0 = wave * 4; t0 < p.T; t0 += 16) {
                const int t = t0 + (lane >> 4);
                if (t < p.T) {
                    int eg;
                    float wt;
                    route_token<16, PL>(p.logits + (size_t)t * p.E_g, p.E_g, p.top_k, n16, eg, wt);
                    if (n16 < p.top_k) {
                        const int sl = t * p.top_k + n16;
                        const int le = eg - p.begin;
                        const int loc = (le >= 0 && le < E) ? le : -1;
                        s_loc[sl] = loc;
                        if (blockIdx.x == 0) {
                            p.ids[sl] = eg;
                            p.wts[sl] = wt;
                            p.pres[sl] = loc >= 0 ? sl : -1;
                        }
                    }
                }
            }
        } else {
            for (int sl = tid; sl < S_slots; sl += 256)
                s_loc[sl] = p.pres[sl] >= 0 ? p.ids[sl] - p.begin : -1;
        }
        __syncthreads();
        build_leaders<256>(S_slots, E, s_loc, s_first, s_lead, s_nlead);
        total_items = s_nlead[0] * nblocks;
    }
    const int G = p.K / kGroup;
    const int nseg = G / KSEG;                         // host guarantees KSEG | G
    const uint32_t row_bytes = (uint32_t)(p.K >> 1);
    // staging: thread -> 16 bytes (8 K positions) of one token of a group:
    // token st_tok, chunk st_c16 = 4*kq + step of the MFMA fragment layout
    const int st_tok = tid >> 4;
    const int st_c16 = tid & 15;
    const int st_idx = (st_c16 & 3) * 64 + act_slot(st_c16 & 3, st_tok + 16 * (st_c16 >> 2));
    int rd_idx[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        rd_idx[i] = i * 64 + act_slot(i, lane);
    const bf16x8 neg136 = neg136_operand();
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.a, p.a_bytes);
    const uint32_t gstride = group_stride(p);

    // XCD-aware schedule: workgroups are dispatched round-robin over the
    // XCDs (workgroup b runs on XCD b % kXcds), each with its own L2. XCD x
    // takes the x-th contiguous share of the chunk-major item list, so the
    // blocks of one chunk, which read the same activation rows, meet in one
    // L2 instead of fetching them once per XCD. The host makes the grid a
    // multiple of kXcds whenever it is at least kXcds.
    // epilogue geometry (bf16 rows through LDS): lane -> (block, row, 16-byte part)
    constexpr int EPI_COLS = KIND == MOE_GEMM_W13_SWIGLU ? 8 : 16;
    constexpr int EPI_LPR = EPI_COLS * 2 / 16;          // lanes per output row
    // with NSUB | (blocks per pass) a lane stores the same subtile row in every pass
    constexpr bool EPI_ONE_ROW = (64 / (16 * EPI_LPR)) % NSUB == 0;
    const int epi_m = ((lane / (16 * EPI_LPR)) % NSUB) * 16 + ((lane / EPI_LPR) & 15);
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(p.c_row_index, p.c_row_bytes);
    const int nx = (int)gridDim.x >= kXcds ? kXcds : 1;
    const int xcd = blockIdx.x % nx;
    const int i_end = (int)((long long)total_items * (xcd + 1) / nx);
    for (int item = (int)((long long)total_items * xcd / nx) + blockIdx.x / nx; item < i_end;
         item += gridDim.x / nx) {
        const int chunk = item / nblocks;
        const int block = item - chunk * nblocks;
        int e, row0, nvalid;
        uint64_t m0 = 0, m1 = 0;                          // small batch: the expert's slots
        if constexpr (CHUNKED) {
            e = uniform(chunk_expert_wave(s_prefix, E, chunk, lane));
            row0 = uniform(s_off[e] + (chunk - s_prefix[e]) * CS);
            nvalid = uniform(min(CS, s_off[e + 1] - row0));
        } else {
            e = uniform(s_loc[s_lead[chunk]]);
            m0 = __ballot(lane < S_slots && s_loc[lane] == e);
            m1 = __ballot(64 + lane < S_slots && s_loc[64 + lane] == e);
            row0 = 0;
            nvalid = uniform(__popcll(m0) + __popcll(m1));
        }
        const int nsub = (nvalid + 15) >> 4;
        const int tile0 = block * BT + wave * TPW;
        const __amdgpu_buffer_rsrc_t rw = make_rsrc(expert_codes(p, e, (uint32_t)p.N * row_bytes), (uint32_t)p.N * row_bytes);
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(expert_scales(p, e, (uint32_t)p.N * G), (uint32_t)p.N * G * 2);

        uint32_t voff_w[TPW], voff_s[TPW];
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            const uint32_t row = (uint32_t)tile_row<KIND>(p, tile0 + t, n16);
            voff_w[t] = code_offset(p, tile0 + t, row, G, row_bytes, lane);
            voff_s[t] = row * (uint32_t)G * 2;
        }
        // output row of the one result row this lane stores in the LDS
        // epilogue, read now (no load under a branch; zeros when unused);
        // small batch: that row's slot
        int32_t c_row;
        if constexpr (CHUNKED)
            c_row = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(rc, (uint32_t)(row0 + min(epi_m, nvalid - 1)) * 4u,
                                                                  0, 0);
        else
            c_row = nth_slot(m0, m1, min(epi_m, nvalid - 1));
        uint32_t voff_x[NSUB];
#pragma unroll
        for (int sb = 0; sb < NSUB; ++sb) {
            const int m = sb * 16 + st_tok;
            uint32_t src;
            if constexpr (SRC == SRC_OFFSETS) {
                const int r = row0 + min(m, nvalid - 1);   // always a valid row: no branch around the load
                src = p.a_row_index ? (uint32_t)(p.a_row_index[r] / p.top_k) : (uint32_t)r;
            } else if constexpr (SRC == SRC_IDS) {
                src = (uint32_t)(s_row[row0 + min(m, nvalid - 1)] / p.top_k);   // the row's token
            } else {
                // row m of the expert is its m-th slot: gate/up reads that
                // slot's token, down reads the slot's own h row
                const int sl = nth_slot(m0, m1, min(m, nvalid - 1));
                src = SRC == SRC_ROUTE ? (uint32_t)(sl / p.top_k) : (uint32_t)sl;
            }
            voff_x[sb] = (m < nvalid) ? src * (uint32_t)p.K * 2 + st_c16 * 16 : kOutOfRange;
        }

        floatx4 tot[TPW][NSUB];
#pragma unroll
        for (int t = 0; t < TPW; ++t)
#pragma unroll
            for (int sb = 0; sb < NSUB; ++sb)
                tot[t][sb] = floatx4{0.f, 0.f, 0.f, 0.f};

        u32x4 xr[KSEG][NSUB];
        u32x4 wv[RING][TPW];                  // weights of groups g .. g+RING-1
        uint32_t sv[2][TPW][SD];              // scales of the current and next segment

        // Activations and scales of segment `seg` into xr / sv[buf]; the
        // segment after the last is read out of range (zeros, no traffic).
        auto load_seg = [&](int seg, auto bufc) {
            constexpr int buf = decltype(bufc)::value;
            const uint32_t oor = seg < nseg ? 0u : kOutOfRange;
            const uint32_t sg = (uint32_t)(seg < nseg ? seg : 0);
#pragma unroll
            for (int j = 0; j < KSEG; ++j)
#pragma unroll
                for (int sb = 0; sb < NSUB; ++sb)
                    xr[j][sb] = bload16(ra, (voff_x[sb] | oor) + j * kGroup * 2, sg * KSEG * kGroup * 2);
            // KSEG == 1: the dword of groups (seg & ~1, seg | 1); seg has the parity of buf
            const uint32_t s_soff = KSEG == 1 ? (sg & ~1u) * 2 : sg * KSEG * 2;
#pragma unroll
            for (int t = 0; t < TPW; ++t)
#pragma unroll
                for (int h = 0; h < SD; ++h)
                    sv[buf][t][h] = __builtin_amdgcn_raw_buffer_load_b32(rs, (voff_s[t] | oor) + h * 4, s_soff, 0);
        };
        auto write_act = [&](auto bufc) {
            constexpr int buf = decltype(bufc)::value;
            u32x4 *dst = &s_act[buf][0][0][0][0];
            // a branch on the layout, not a select: with tiled codes the
            // fragments are stored as loaded and no permutation is formed
            if (p.w_tiled) {
#pragma unroll
                for (int j = 0; j < KSEG; ++j)
#pragma unroll
                    for (int sb = 0; sb < NSUB; ++sb)
                        dst[(j * NSUB + sb) * 256 + st_idx] = xr[j][sb];
            } else {
#pragma unroll
                for (int j = 0; j < KSEG; ++j)
#pragma unroll
                    for (int sb = 0; sb < NSUB; ++sb)
                        xr[j][sb] = permute_act(xr[j][sb]);
                asm volatile("" ::: "memory");   // keeps the two store sequences apart
#pragma unroll
                for (int j = 0; j < KSEG; ++j)
#pragma unroll
                    for (int sb = 0; sb < NSUB; ++sb)
                        dst[(j * NSUB + sb) * 256 + st_idx] = xr[j][sb];
            }
        };
        auto load_w = [&](int g, int b) {
            const uint32_t oor = g < G ? 0u : kOutOfRange;
            const uint32_t soff = (uint32_t)(g < G ? g : 0) * gstride;
#pragma unroll
            for (int t = 0; t < TPW; ++t)
                wv[b][t] = bload16_codes<NT>(rw, voff_w[t] | oor, soff);
        };
        // One group: the -136*sum(x) chain per subtile, then every tile's
        // chain of 4 MFMAs starting from it; the group scale is applied to
        // the chain result.
        auto compute = [&](auto bufc, int j, int b) {
            constexpr int buf = decltype(bufc)::value;
            const u32x4 *src = &s_act[buf][0][0][0][0];
#pragma unroll
            for (int sb = 0; sb < NSUB; ++sb) {
                if (sb < nsub) {
                    u32x4 a[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        a[i] = src[(j * NSUB + sb) * 256 + rd_idx[i]];
                    floatx4 corr = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        corr = mfma(a[i], neg136, corr);
                    // tile t's scale FMAs go out among tile t + 1's MFMAs
                    // and stay in this group (no sinking past the loads
                    // that follow), so only the last tile's trail it
                    floatx4 accp = corr;
                    float scp = 0.f;
#pragma unroll
                    for (int t = 0; t < TPW; ++t) {
                        floatx4 acc = corr;
                        acc = mfma(a[0], unpack8(wv[b][t].x), acc);
                        acc = mfma(a[1], unpack8(wv[b][t].y), acc);
                        acc = mfma(a[2], unpack8(wv[b][t].z), acc);
                        acc = mfma(a[3], unpack8(wv[b][t].w), acc);
                        if (t > 0) {
                            tot[t - 1][sb].x = __builtin_fmaf(scp, accp.x, tot[t - 1][sb].x);
                            tot[t - 1][sb].y = __builtin_fmaf(scp, accp.y, tot[t - 1][sb].y);
                            tot[t - 1][sb].z = __builtin_fmaf(scp, accp.z, tot[t - 1][sb].z);
                            tot[t - 1][sb].w = __builtin_fmaf(scp, accp.w, tot[t - 1][sb].w);
                        }
                        const uint32_t d = sv[buf][t][j >> 1];
                        const int hi = KSEG == 1 ? buf : (j & 1);
                        scp = __uint_as_float(hi ? (d & 0xFFFF0000u) : (d << 16));
                        accp = acc;
                    }
                    tot[TPW - 1][sb].x = __builtin_fmaf(scp, accp.x, tot[TPW - 1][sb].x);
                    tot[TPW - 1][sb].y = __builtin_fmaf(scp, accp.y, tot[TPW - 1][sb].y);
                    tot[TPW - 1][sb].z = __builtin_fmaf(scp, accp.z, tot[TPW - 1][sb].z);
                    tot[TPW - 1][sb].w = __builtin_fmaf(scp, accp.w, tot[TPW - 1][sb].w);
#pragma unroll
                    for (int t = 0; t < TPW; ++t)
                        asm volatile("" : "+v"(tot[t][sb]));
                }
            }
        };
        // Segment `seg` staged in buffer BUF: prefetch the next segment,
        // run its groups, stage the next segment into the other buffer.
        // BUF is a constant so that register double buffers are indexed
        // statically (no selects).
        auto segment = [&](auto bufc, int seg) {
            constexpr int buf = decltype(bufc)::value;
            __syncthreads();                              // segment seg staged; the other buffer free
            load_seg(seg + 1, std::integral_constant<int, buf ^ 1>());
#pragma unroll
            for (int j = 0; j < KSEG; ++j) {
                const int g = seg * KSEG + j;
                load_w(g + RING - 1, (buf * KSEG + j + RING - 1) % RING);
                compute(bufc, j, (buf * KSEG + j) % RING);
            }
            if (seg + 1 < nseg)
                write_act(std::integral_constant<int, buf ^ 1>());
        };

        __syncthreads();                                  // previous item done with s_act
        load_seg(0, std::integral_constant<int, 0>());
#pragma unroll
        for (int r = 0; r < RING - 1; ++r)
            load_w(r, r);
        write_act(std::integral_constant<int, 0>());
        int seg = 0;
        for (; seg + 2 <= nseg; seg += 2) {
            segment(std::integral_constant<int, 0>(), seg);
            segment(std::integral_constant<int, 1>(), seg + 1);
        }
        if (seg < nseg)
            segment(std::integral_constant<int, 0>(), seg);

        // ---- epilogue: bf16 results pass through the LDS buffer the last
        // segment did not use (every wave is past that segment's barrier), so
        // each lane stores one 16-byte run of an output row instead of four
        // scattered 2-byte values ----
        constexpr bool SWI = KIND == MOE_GEMM_W13_SWIGLU;
        constexpr int COLS = SWI ? 8 : 16;                 // output columns per tile
        constexpr int NBLK = TPW * NSUB;                   // (tile, subtile) blocks of a wave
        constexpr bool VIA_LDS = 4 * NBLK * 16 * COLS * 2 <= KSEG * NSUB * 4096;
        if (VIA_LDS && (SWI || !p.c_f32)) {
            uint16_t *so = reinterpret_cast<uint16_t *>(&s_act[nseg & 1][0][0][0][0]) + wave * (NBLK * 16 * COLS);
#pragma unroll
            for (int t = 0; t < TPW; ++t)
#pragma unroll
                for (int sb = 0; sb < NSUB; ++sb) {
                    const floatx4 v = tot[t][sb];
                    const float r4[4] = {v.x, v.y, v.z, v.w};
                    if (SWI) {
                        // lane n16 < 8 holds the gate row of feature n16 for
                        // token rows 4 kq + 0..3, lane n16 + 8 the up row: the
                        // gate lane forms rows 0 and 1 (it receives two up
                        // values), the up lane rows 2 and 3 (two gate values),
                        // so every lane stores and none waits on a branch
                        const bool gl = n16 < 8;
#pragma unroll
                        for (int j = 0; j < 2; ++j) {
                            const float recv = row_swap8(gl ? r4[j + 2] : r4[j]);
                            const float gate = gl ? r4[j] : recv, up = gl ? recv : r4[j + 2];
                            const int rr = kq * 4 + (gl ? j : j + 2);
                            so[((t * NSUB + sb) * 16 + rr) * COLS + (n16 & 7)] =
                                (uint16_t)f32_to_bf16_rne(silu_fast(gate) * up);
                        }
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            so[((t * NSUB + sb) * 16 + kq * 4 + i) * COLS + n16] = (uint16_t)f32_to_bf16_rne(r4[i]);
                    }
                }
            __builtin_amdgcn_wave_barrier();
            uint16_t *c = static_cast<uint16_t *>(p.c);
            constexpr int LPR = COLS * 2 / 16;                 // lanes per row (16 bytes each)
            constexpr int BPP = 64 / (16 * LPR);               // blocks per pass
#pragma unroll
            for (int b0 = 0; b0 < NBLK; b0 += BPP) {
                const int b = b0 + lane / (16 * LPR);
                const int rr = (lane / LPR) & 15;
                const int part = lane % LPR;
                const int t = b / NSUB, sb = b - (b / NSUB) * NSUB;
                const int m = sb * 16 + rr;
                if (b < NBLK && sb < nsub && m < nvalid) {
                    const u32x4 d = *reinterpret_cast<const u32x4 *>(so + (b * 16 + rr) * COLS + part * 8);
                    const int orow = !CHUNKED ? c_row
                                     : !p.c_row_index ? row0 + m : (EPI_ONE_ROW ? c_row : p.c_row_index[row0 + m]);
                    *reinterpret_cast<u32x4 *>(c + (size_t)orow * p.ldc + (tile0 + t) * COLS + part * 8) = d;
                }
            }
        } else {
#pragma unroll
            for (int t = 0; t < TPW; ++t)
#pragma unroll
                for (int sb = 0; sb < NSUB; ++sb)
                    if (sb < nsub)
                        store_tile<KIND>(p, tot[t][sb], tile0 + t, row0, sb * 16 + kq * 4, nvalid, n16);
        }
    }
}

// ---------------------------------------------------------------------------
// gemm_splitk_kernel: one 16-row tile per workgroup, K split over NWAVES
// waves (contiguous group ranges), LDS reduction in wave order. For about one
// row per active expert: activations come straight from global memory.
// ---------------------------------------------------------------------------
template <int KIND, int NWAVES, int GB>
__global__ __launch_bounds__(NWAVES * 64) void gemm_splitk_kernel(GemmArgs p)
{
    constexpr int CS = 16;
    __shared__ int s_prefix[kMaxExperts + kMaxSharedExperts + 1];   // routed + shared experts
    __shared__ int s_wtot[NWAVES];
    __shared__ floatx4 s_red[NWAVES][64];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int n16 = lane & 15;
    const int kq = lane >> 4;
    const int E = p.num_experts;
    build_chunk_prefix<NWAVES * 64>(p.offsets, p.dense_rows, E, CS, s_prefix, s_wtot);

    const int ntiles = p.N >> 4;
    const int total_items = s_prefix[E] * ntiles;
    const int G = p.K / kGroup;
    int g0, g1;
    splitk_groups(wave, G, NWAVES, g0, g1);
    const uint32_t row_bytes = (uint32_t)(p.K >> 1);
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.a, p.a_bytes);
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(p.c_row_index, p.c_row_bytes);
    const uint32_t gstride = group_stride(p);

    for (int item = blockIdx.x; item < total_items; item += gridDim.x) {
        const int chunk = item / ntiles;
        const int tile = item - chunk * ntiles;
        const int e = uniform(chunk_expert_wave(s_prefix, E, chunk, lane));
        const int row0 = uniform(expert_offset(p.offsets, p.dense_rows, e) + (chunk - s_prefix[e]) * CS);
        const int nvalid = uniform(min(CS, expert_offset(p.offsets, p.dense_rows, e + 1) - row0));
        const __amdgpu_buffer_rsrc_t rw = make_rsrc(expert_codes(p, e, (uint32_t)p.N * row_bytes), (uint32_t)p.N * row_bytes);
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(expert_scales(p, e, (uint32_t)p.N * G), (uint32_t)p.N * G * 2);
        const uint32_t row = (uint32_t)tile_row<KIND>(p, tile, n16);
        const uint32_t voff_w = code_offset(p, tile, row, G, row_bytes, lane);
        const uint32_t voff_s = row * (uint32_t)G * 2;
        int c_rows[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            c_rows[i] = (int)__builtin_amdgcn_raw_buffer_load_b32(
                rc, (uint32_t)(row0 + min(kq * 4 + i, nvalid - 1)) * 4u, 0, 0);
        uint32_t voff_x = kOutOfRange;
        if (n16 < nvalid) {
            const int r = row0 + n16;
            const uint32_t src = p.a_row_index ? (uint32_t)(p.a_row_index[r] / p.top_k) : (uint32_t)r;
            voff_x = src * (uint32_t)p.K * 2 + kq * 64;
        }
        const floatx4 tot = splitk_wave_sum<GB>(rw, voff_w, gstride, rs, voff_s, ra, voff_x, g0, g1, p.w_tiled != 0);
        const floatx4 sum = splitk_reduce<NWAVES>(tot, s_red, wave, lane);
        if (wave == 0)
            store_tile<KIND>(p, sum, tile, row0, kq * 4, nvalid, n16, c_rows);
    }
}

// ---------------------------------------------------------------------------
// gemm_tile_kernel: many rows per expert (prefill). One workgroup of 8 waves
// per CU owns an item = (chunk of up to 64 rows of one expert, block of 8 x 4
// sixteen-row tiles); wave w computes all four 16-token subtiles of its 4
// tiles, so each unpacked code fragment feeds up to 4 MFMAs.
//  * Both operands reach LDS through the buffer unit's LDS-DMA (no
//    registers, no staging instructions), three 128-wide groups deep: the
//    activations of a group (64 rows x 256 bytes, shared by the 8 waves) and
//    each wave's own codes (4 tiles x 1 KiB). With two groups in flight the
//    latency of a code fetch that misses L2 stays hidden. A group's copies
//    are waited for with an explicit vmcnt (every group issues the same 6
//    copies, so the count is a constant) and a bare s_barrier (a
//    __syncthreads fence would wait for every copy in flight).
//  * Rows past the chunk are read out of range (zeros).
//  * Scales: each lane loads the scales of groups 4kq .. 4kq+3 of its row
//    once per item; a group's scale is fetched from the owning lane with
//    ds_bpermute.
//  * The +136 offset is removed once per item instead of once per group and
//    tile: per group, waves w and w+4 add 136 * sum(x) of subtile w's two
//    halves of K to column g of one MFMA tile (operand B one-hot on column
//    g), and after the last group two MFMAs per (subtile, tile) add
//    sum_g s[n][g] * (-136 * sum_g x), each sum split exactly into three
//    bf16 terms (hi + mid + lo). Needs G <= 16 (one column per group).
//  * Tiled codes only: they unpack in column order, matching the
//    activations as they lie in memory.
// ---------------------------------------------------------------------------
// Tile kernel shapes: WAVES waves, NS 16-row subtiles per item (4 * NS
// activation copies per group, two per wave). 8 x 4: one workgroup per CU
// (prefill); 4 x 2: two per CU (32-row chunks).
constexpr int kTileStages = 3;
constexpr int tile_act_bytes(int NS) { return NS * 4 * 64 * 16; }         // one group's activation fragments
constexpr int tile_code_bytes(int WAVES) { return WAVES * 4 * 1024; }    // one group: 4 tiles x 1 KiB per wave
constexpr int tile_sx_bytes(int WAVES) { return WAVES * 16 * 16 * 4; }
constexpr int tile_chunk_table(int WAVES) { return WAVES == 8 ? 1024 : 256; }   // chunk -> expert entries in LDS
constexpr size_t tile_lds_bytes(int WAVES, int NS, int E)
{
    return (size_t)kTileStages * (tile_act_bytes(NS) + tile_code_bytes(WAVES)) + tile_sx_bytes(WAVES) +
           sizeof(int) * (2 * (E + 1) + WAVES + 64 + tile_chunk_table(WAVES));
}

// fp32 pair -> bf16 pair, round to nearest even (v_cvt_pk_bf16_f32; fp32
// denormals are kept, so this is the IEEE rounding for every finite value)
__device__ __forceinline__ uint32_t bf16_pair(float lo, float hi)
{
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2{lo, hi}), b2));
}

constexpr uint32_t vmcnt_imm(int n)                   // s_waitcnt vmcnt(n), other counters untouched
{
    return (uint32_t)((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <int KIND, int kTileWaves, int NS>
__global__ __launch_bounds__(kTileWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void gemm_tile_kernel(GemmArgs p)
{
    constexpr int TPW = 4;                              // tiles per wave
    static_assert(4 * NS == 2 * kTileWaves, "two activation copies per wave and group");
    constexpr int CS = 16 * NS;                         // rows per item
    constexpr int kTileActBytes = tile_act_bytes(NS);
    constexpr int kTileCodeBytes = tile_code_bytes(kTileWaves);
    constexpr int kTileSxBytes = tile_sx_bytes(kTileWaves);
    constexpr int kTileChunkTable = tile_chunk_table(kTileWaves);
    constexpr int BT = kTileWaves * TPW;                // tiles per block
    constexpr int NCOPY = 2 + TPW;                      // copies a wave issues per group
    extern __shared__ __align__(16) unsigned char s_dyn[];
    u32x4 *s_a = reinterpret_cast<u32x4 *>(s_dyn);                                  // [stage][copy][lane]
    u32x4 *s_w = reinterpret_cast<u32x4 *>(s_dyn + kTileStages * kTileActBytes);   // [stage][wave][tile][lane]
    float *s_sx = reinterpret_cast<float *>(s_dyn + kTileStages * (kTileActBytes + kTileCodeBytes));
    const int E = p.num_experts;
    int *s_prefix = reinterpret_cast<int *>(s_dyn + kTileStages * (kTileActBytes + kTileCodeBytes) + kTileSxBytes);
    int *s_off = s_prefix + (E + 1);
    int *s_wtot = s_off + (E + 1);
    int *s_crow = s_wtot + kTileWaves;                 // output row of each of the item's 64 rows
    int *s_chunk_e = s_crow + 64;                      // expert of each chunk (when they fit)

    const int tid = threadIdx.x;
    const int wave = uniform(tid >> 6);                // scalar: wave-dependent choices are branches
    // The lane index and what derives from it are re-formed at the start of
    // every item, behind an empty asm statement: the compiler then forms the
    // lane-dependent addresses where they are used instead of hoisting them
    // out of the item loop, where they would hold registers throughout (and
    // spill, each reload waiting for every load in flight).
    int lane = tid & 63, n16 = lane & 15, kq = lane >> 4;
    int m_act = 16 * (wave >> 1) + n16;                // this lane's activation row in an item
    auto refresh_lane = [&]() {
        asm volatile("" : "+v"(lane));
        n16 = lane & 15;
        kq = lane >> 4;
        m_act = 16 * (wave >> 1) + n16;
    };
    build_chunk_prefix<kTileWaves * 64>(p.offsets, p.dense_rows, E, CS, s_prefix, s_wtot, s_off);

    const int ntiles = p.N >> 4;
    const int nblocks = ntiles / BT;
    const int total_items = s_prefix[E] * nblocks;
    const int G = p.K / kGroup;
    const uint32_t row_bytes = (uint32_t)(p.K >> 1);
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.a, p.a_bytes);
    const __amdgpu_buffer_rsrc_t ri = make_rsrc(p.a_row_index, p.a_row_bytes);
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(p.c_row_index, p.c_row_bytes);
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(p.c, p.c_bytes);
    typedef __attribute__((address_space(3))) unsigned char lds_byte;

    // Epilogue: a wave's bf16 results pass through its own 4 KiB of the
    // codes of the item's last stage (64 rows x OCOLS columns, in HALVES
    // passes), then each store writes whole row runs of OCOLS * 2 bytes (LPR
    // lanes of 16 bytes per row, RPP rows per store).
    constexpr bool SWI = KIND == MOE_GEMM_W13_SWIGLU;
    constexpr int COLS = SWI ? 8 : 16;                  // output columns per tile
    constexpr int HALVES = SWI ? 1 : 2;
    constexpr int TH = TPW / HALVES;                    // tiles per pass
    constexpr int OCOLS = TH * COLS;
    constexpr int LPR = OCOLS * 2 / 16;
    constexpr int RPP = 64 / LPR;
    constexpr int NST = HALVES * (CS / RPP);            // stores per wave and item, always issued
    static_assert(CS * OCOLS * 2 <= TPW * 1024, "a pass fits the wave's codes of one stage");

    const int nx = (int)gridDim.x >= kXcds ? kXcds : 1;
    const int xcd = blockIdx.x % nx;
    const int i_end = (int)((long long)total_items * (xcd + 1) / nx);
    const int i_beg = (int)((long long)total_items * xcd / nx) + blockIdx.x / nx;
    const int i_step = gridDim.x / nx;

    // ---- item geometry (all uniform) ----
    struct Geo {
        int e, row0, nvalid, tile0;
    };
    // the expert of every chunk, looked up once here instead of a binary
    // search at every item (the search stays for more chunks than the table)
    const bool chunk_table = s_prefix[E] <= kTileChunkTable;
    if (chunk_table) {
        for (int c = tid; c < s_prefix[E]; c += kTileWaves * 64)
            s_chunk_e[c] = chunk_expert(s_prefix, E, c);
        __syncthreads();
    }
    auto geo = [&](int it) {
        Geo q;
        const int ch = it / nblocks;
        const int block = it - ch * nblocks;
        q.e = uniform(chunk_table ? s_chunk_e[ch] : chunk_expert(s_prefix, E, ch));
        q.row0 = uniform(s_off[q.e] + (ch - s_prefix[q.e]) * CS);
        q.nvalid = uniform(min(CS, s_off[q.e + 1] - q.row0));
        q.tile0 = block * BT + wave * TPW;
        return q;
    };
    // gather index of that row (the row itself without one): one load, always
    // issued (with no index its buffer holds 0 bytes and the load returns 0)
    auto load_src = [&](const Geo &q) -> int {
        const int r = q.row0 + min(m_act, q.nvalid - 1);
        return (int)__builtin_amdgcn_raw_buffer_load_b32(ri, (uint32_t)r * 4u, 0, 0) + (p.a_row_index ? 0 : r);
    };
    auto act_offset = [&](const Geo &q, int src, bool valid) -> uint32_t {
        const uint32_t s = p.a_row_index ? (uint32_t)(src / p.top_k) : (uint32_t)src;
        return (valid && m_act < q.nvalid) ? s * (uint32_t)p.K * 2 + (uint32_t)kq * 64 : kOutOfRange;
    };
    auto codes_rsrc = [&](const Geo &q) {
        return make_rsrc(expert_codes(p, q.e, (uint32_t)p.N * row_bytes), (uint32_t)p.N * row_bytes);
    };
    // this lane's scales of groups 4kq .. 4kq+3 for each tile, and the row
    // index entry of the item's row `lane` (0 without an index; the output
    // row is this plus row0 + lane then): TPW + 1 loads
    auto load_item_rows = [&](const Geo &q, bool valid, u32x2 (&sc)[TPW], int &crow) {
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(expert_scales(p, q.e, (uint32_t)p.N * G), (uint32_t)p.N * G * 2);
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            const uint32_t row = (uint32_t)tile_row<KIND>(p, q.tile0 + t, n16);
            const uint32_t vs = valid ? row * (uint32_t)G * 2 + kq * 8 : kOutOfRange;
            sc[t] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, vs, 0, 0));
        }
        crow = (int)__builtin_amdgcn_raw_buffer_load_b32(rc, (uint32_t)(q.row0 + min(lane, q.nvalid - 1)) * 4u, 0, 0);
    };

    // Group g of an item -> stage st: 2 activation copies, and this wave's 4
    // code copies (issued separately: the codes sit in the wave's own part of
    // the stage, which it refills as soon as it has read it). Lane l's 16
    // bytes land at the LDS pointer + 16 l (the instruction's immediate
    // offset would move the LDS side too; it stays 0, and the step's 16-byte
    // column offset is a scalar offset).
    // Activation copy q = 2 wave + j (j < 2) is MFMA fragment (subtile q / 4,
    // step q % 4) of the group: lane (n16, kq) brings the 16 bytes it will
    // read, chunk 4 kq + q % 4 of token 16 (q / 4) + n16 (MFMA step i of lane
    // (n16, kq) multiplies K = 32 kq + 8 i .. +8 of the group: a lane's 16
    // code bytes hold K = 32 kq .. +32, one word per step).
    auto copy_act = [&](uint32_t voff_a, int g, int st) {
        const uint32_t soff = (uint32_t)g * (kGroup * 2) + (uint32_t)(wave & 1) * 32;
        lds_byte *da = (lds_byte *)(s_a + (st * 4 * NS + 2 * wave) * 64);
#pragma unroll
        for (int j = 0; j < 2; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, da + j * 1024, 16, voff_a, soff + j * 16, 0, 0);
    };
    // (the tile's place in the tiled layout is a scalar offset: one lane
    // offset register serves every copy)
    auto copy_codes = [&](__amdgpu_buffer_rsrc_t rw, int tile0, bool valid, int g, int st) {
        lds_byte *dw = (lds_byte *)(s_w + ((st * kTileWaves + wave) * TPW) * 64);
        const uint32_t vo = valid ? (uint32_t)lane * 16u : kOutOfRange;
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            const int tl = tile0 + t;
            const uint32_t so = (uint32_t)((tl >> 3) * G * 8 + (tl & 7)) * 1024u + (uint32_t)g * 8192u;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, dw + t * 1024, 16, vo, so, 0, 0);
        }
    };
    auto wait_barrier = [&](auto vm) {                  // s_waitcnt vmcnt(vm) lgkmcnt(0); s_barrier
        constexpr uint32_t W = vmcnt_imm(decltype(vm)::value) & 0xF0FFu;
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(W);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_barrier();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_sched_barrier(0);
    };
    using I0 = std::integral_constant<int, 0>;

    // Pipeline across items. The copies of groups 0 and 1 of the next item
    // go out during this item's groups G-3 and G-2 (into the stages those
    // free), its scales and output rows at this item's start, its group 2
    // after this item's epilogue (whose staging used that stage). Every item
    // issues the same loads and stores, in the same order, per wave:
    //   [gather index two items on] [next: TPW scale loads, 1 row load]
    //   [its group 2] [its groups 3 .. G-1] [next: group 0] [next: group 1]
    //   [NST stores] | wait for all but the stores, barrier | ...
    // (an item with no next item issues those copies and loads out of
    // range), so each wait below is an exact compile-time count: before
    // group 0, NCOPY + NST + TPW + 2 + NCOPY later loads and stores; before
    // group 1, NST + TPW + 2 + NCOPY; later, one group's NCOPY. Each item's
    // loads of scales, rows and gather indices are complete before the item
    // starts, as the compiler can see.
    u32x2 csc[TPW], csc_n[TPW];                         // scales of this item and the next
    int crow = 0, crow_n = 0;                           // output-row entries of this item and the next
    int src_cur = 0, src_n1 = 0;                        // gather indices of this item and the next
    Geo q_cur{0, 0, 1, 0}, q_nxt{0, 0, 1, 0};
    if (i_beg < i_end) {
        q_cur = geo(i_beg);
        q_nxt = geo(min(i_beg + i_step, i_end - 1));
        src_cur = load_src(q_cur);
        src_n1 = load_src(q_nxt);
        load_item_rows(q_cur, true, csc, crow);
        {
            constexpr uint32_t W0 = vmcnt_imm(0);
            __builtin_amdgcn_s_waitcnt(W0);
        }
        const uint32_t va = act_offset(q_cur, src_cur, true);
        const __amdgpu_buffer_rsrc_t rw = codes_rsrc(q_cur);
        __builtin_amdgcn_sched_barrier(0);
        copy_act(va, 0, 0);
        copy_codes(rw, q_cur.tile0, true, 0, 0);
        copy_act(va, 1, 1);
        copy_codes(rw, q_cur.tile0, true, 1, 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < NST; ++j)                   // in place of a previous item's stores
            __builtin_amdgcn_raw_buffer_store_b128(u32x4{0u, 0u, 0u, 0u}, ro, kOutOfRange, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
    }
    int st0 = 0;                                        // stage of the item's group 0
    for (int item = i_beg; item < i_end; item += i_step) {
        refresh_lane();
        const Geo q = q_cur, qn = q_nxt;                 // qn: this item again when it is the last
        const Geo qnn = geo(min(item + 2 * i_step, i_end - 1));
        const int nsub = (q.nvalid + 15) >> 4;
        const __amdgpu_buffer_rsrc_t rw = codes_rsrc(q);
        const uint32_t voff_a = act_offset(q, src_cur, true);
        const bool has_next = item + i_step < i_end;
        const __amdgpu_buffer_rsrc_t rwn = codes_rsrc(qn);
        const uint32_t voff_an = act_offset(qn, src_n1, has_next);
        const int st2 = st0 == 0 ? 2 : st0 - 1;        // stage of group 2
        const int st_last = (st0 + G - 1) % 3;

        __builtin_amdgcn_sched_barrier(0);
        const int src_n2 = load_src(qnn);               // used two items on
        load_item_rows(qn, has_next, csc_n, crow_n);    // used by the next item
        __builtin_amdgcn_sched_barrier(0);
        copy_act(voff_a, 2, st2);
        copy_codes(rw, q.tile0, true, 2, st2);
        __builtin_amdgcn_sched_barrier(0);

        floatx4 tot[TPW][NS];
#pragma unroll
        for (int t = 0; t < TPW; ++t)
#pragma unroll
            for (int sb = 0; sb < NS; ++sb)
                tot[t][sb] = floatx4{0.f, 0.f, 0.f, 0.f};
        floatx4 sxacc = {0.f, 0.f, 0.f, 0.f};

        // The group pipeline, NSV valid subtiles (a compile-time count: the
        // MFMA chains of a group are one branch-free block). Iteration g:
        //   wait for this wave's activation reads of group g and its copies
        //   of group g + 1; barrier (every wave has group g's activations in
        //   registers, so their part of stage st is free, and every copy of
        //   group g + 1 has landed); start the activation copies of group
        //   g + 3 (or of the next item's group g + 3 - G); compute group g,
        //   reading this wave's codes of stage st; refill that part with the
        //   matching codes; read group g + 1's activations.
        // Waves read right after their own compute, not all at once after a
        // barrier, so the LDS reads of the 8 waves spread out.
        auto groups = [&](auto nsc) {
            constexpr int NSV = decltype(nsc)::value;
            u32x4 a[NSV][4];
            auto read = [&](int st) {
                const u32x4 *src = s_a + st * 4 * NS * 64 + lane;
#pragma unroll
                for (int sb = 0; sb < NSV; ++sb)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        a[sb][i] = src[(4 * sb + i) * 64];
            };
            auto compute = [&](int g, int st) {
                // 136 * sum(x) of subtile wave % NS, steps 2 (wave / NS) .. +1, into column g
                const uint32_t oh = n16 == g ? 0x43084308u : 0u;
                const bf16x8 ohv = __builtin_bit_cast(bf16x8, u32x4{oh, oh, oh, oh});
#pragma unroll
                for (int w = 0; w < NSV; ++w) {
                    if (wave % NS == w) {
                        if (wave < NS) {
                            sxacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[w][0]), ohv, sxacc, 0, 0, 0);
                            sxacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[w][1]), ohv, sxacc, 0, 0, 0);
                        } else {
                            sxacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[w][2]), ohv, sxacc, 0, 0, 0);
                            sxacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[w][3]), ohv, sxacc, 0, 0, 0);
                        }
                    }
                }
                const u32x4 *wsrc = s_w + ((st * kTileWaves + wave) * TPW) * 64 + lane;
                const int src_lane = 4 * (n16 + 16 * (g >> 2));  // lane holding this row's scale of group g
                // tile t + 1's codes and scale are read while tile t computes
                u32x4 w_next = wsrc[0];
                uint32_t sd_next = __builtin_amdgcn_ds_bpermute(src_lane, (int)((g & 2) ? csc[0].y : csc[0].x));
                // Tile t's scale FMAs wait for its MFMA chains; they are
                // issued among tile t + 1's MFMAs (the matrix unit runs
                // independent VALU work of the same wave alongside), so only
                // the last tile's FMAs follow the group's last MFMA.
                floatx4 accp[NSV];
                float scp = 0.f;
                auto scale_add = [&](int t) {
#pragma unroll
                    for (int sb = 0; sb < NSV; ++sb) {
                        tot[t][sb].x = __builtin_fmaf(scp, accp[sb].x, tot[t][sb].x);
                        tot[t][sb].y = __builtin_fmaf(scp, accp[sb].y, tot[t][sb].y);
                        tot[t][sb].z = __builtin_fmaf(scp, accp[sb].z, tot[t][sb].z);
                        tot[t][sb].w = __builtin_fmaf(scp, accp[sb].w, tot[t][sb].w);
                    }
                };
#pragma unroll
                for (int t = 0; t < TPW; ++t) {
                    const u32x4 w4 = w_next;
                    const uint32_t sd = sd_next;
                    if (t + 1 < TPW) {
                        w_next = wsrc[(t + 1) * 64];
                        sd_next = __builtin_amdgcn_ds_bpermute(src_lane, (int)((g & 2) ? csc[t + 1].y : csc[t + 1].x));
                    }
                    const float sc = __uint_as_float((g & 1) ? (sd & 0xFFFF0000u) : (sd << 16));
                    const bf16x8 qv[4] = {unpack8(w4.x), unpack8(w4.y), unpack8(w4.z), unpack8(w4.w)};
                    // steps outer, subtiles inner: the NSV chains interleave, so
                    // dependent MFMAs are NSV issues apart
                    floatx4 acc[NSV];
#pragma unroll
                    for (int sb = 0; sb < NSV; ++sb)
                        acc[sb] = mfma(a[sb][0], qv[0], floatx4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                    for (int i = 1; i < 4; ++i)
#pragma unroll
                        for (int sb = 0; sb < NSV; ++sb)
                            acc[sb] = mfma(a[sb][i], qv[i], acc[sb]);
                    if (t > 0)
                        scale_add(t - 1);
                    // issue order: one MFMA, then up to two VALU instructions
                    // (the previous tile's FMAs, the next tile's unpack)
#pragma unroll
                    for (int i = 0; i < 4 * NSV; ++i) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
                    }
#pragma unroll
                    for (int sb = 0; sb < NSV; ++sb)
                        accp[sb] = acc[sb];
                    scp = sc;
                }
                scale_add(TPW - 1);
                // keep the FMAs here, among this group's MFMAs, instead of
                // letting them sink past the code copies that follow
#pragma unroll
                for (int t = 0; t < TPW; ++t)
#pragma unroll
                    for (int sb = 0; sb < NSV; ++sb)
                        asm volatile("" : "+v"(tot[t][sb]));
            };

            wait_barrier(std::integral_constant<int, 2 * NCOPY + TPW + 2 + NST>());   // group 0 landed
            read(st0);
            int st = st0;
            for (int g = 0; g < G; ++g) {
                if (g == 0)
                    wait_barrier(std::integral_constant<int, NCOPY + TPW + 2 + NST>());   // group 1
                else if (g + 1 < G)
                    wait_barrier(std::integral_constant<int, NCOPY>());             // group g + 1
                else
                    wait_barrier(std::integral_constant<int, 2 * NCOPY>());         // nothing new to land
                const bool own = g + 3 < G, nxt = !own && g + 3 - G < 2;
                if (own)
                    copy_act(voff_a, g + 3, st);
                else if (nxt)
                    copy_act(voff_an, g + 3 - G, st);
                __builtin_amdgcn_sched_barrier(0);
                compute(g, st);
                __builtin_amdgcn_sched_barrier(0);  // this wave's codes of stage st have been read
                if (own)
                    copy_codes(rw, q.tile0, true, g + 3, st);
                else if (nxt)
                    copy_codes(rwn, qn.tile0, has_next, g + 3 - G, st);
                __builtin_amdgcn_sched_barrier(0);
                st = st == 2 ? 0 : st + 1;
                if (g + 1 < G)
                    read(st);
            }
        };
        if (nsub >= NS)
            groups(std::integral_constant<int, NS>());
        else if constexpr (NS == 4) {
            if (nsub == 3)
                groups(std::integral_constant<int, 3>());
            else if (nsub == 2)
                groups(std::integral_constant<int, 2>());
            else
                groups(std::integral_constant<int, 1>());
        } else {
            groups(std::integral_constant<int, 1>());
        }

        // ---- per-item correction: the s_sx sums of every wave (and the
        // output rows) after a barrier that waits for no copy ----
#pragma unroll
        for (int i = 0; i < 4; ++i)
            s_sx[wave * 256 + (kq * 4 + i) * 16 + n16] = sxacc[i];
        if (wave == 0)
            s_crow[lane] = crow + (p.c_row_index ? 0 : q.row0 + lane);
        wait_barrier(std::integral_constant<int, 63>());
        u32x4 bcorr[TPW];                                // B: s[n][4kq + j] twice, j = 0..3
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            uint32_t h[4] = {csc[t].x & 0xFFFFu, csc[t].x >> 16, csc[t].y & 0xFFFFu, csc[t].y >> 16};
#pragma unroll
            for (int j = 0; j < 4; ++j)
                h[j] = (kq * 4 + j < G) ? h[j] * 0x10001u : 0u;
            bcorr[t] = u32x4{h[0], h[1], h[2], h[3]};
        }
#pragma unroll
        for (int sb = 0; sb < NS; ++sb) {
            if (sb < nsub) {
                const floatx4 v0 = *reinterpret_cast<const floatx4 *>(s_sx + sb * 256 + n16 * 16 + kq * 4);
                const floatx4 v1 = *reinterpret_cast<const floatx4 *>(s_sx + (sb + NS) * 256 + n16 * 16 + kq * 4);
                const float vv[4] = {v0.x + v1.x, v0.y + v1.y, v0.z + v1.z, v0.w + v1.w};
                // -136 * sum(x) split into three bf16 terms hi + mid + lo that
                // add up to the binary32 value exactly (each remainder is exact
                // and has at most 8 fewer significant bits than the last), so
                // the correction is as accurate as the per-group one of the
                // streaming kernel whatever the size of sum(x)
                uint32_t d[4], dl[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float nv = -vv[j];
                    const float hi = __uint_as_float(bf16_pair(nv, 0.f) << 16);
                    const float r1 = nv - hi;
                    const float mid = __uint_as_float(bf16_pair(r1, 0.f) << 16);
                    d[j] = bf16_pair(hi, mid);
                    dl[j] = bf16_pair(r1 - mid, 0.f);
                }
                const u32x4 acorr = {d[0], d[1], d[2], d[3]};
                const u32x4 acorr_lo = {dl[0], dl[1], dl[2], dl[3]};
#pragma unroll
                for (int t = 0; t < TPW; ++t) {
                    tot[t][sb] = mfma(acorr, __builtin_bit_cast(bf16x8, bcorr[t]), tot[t][sb]);
                    tot[t][sb] = mfma(acorr_lo, __builtin_bit_cast(bf16x8, bcorr[t]), tot[t][sb]);
                }
            }
        }

        // ---- epilogue: bf16 results pass through this wave's own codes of
        // the last stage, then every store writes whole row runs; a row past
        // the chunk stores out of range (the store count stays fixed). The
        // 16-byte column chunks of row rr sit at chunk position c ^ ((rr / 4)
        // % 4), so the four row quads a write instruction covers fall on
        // different LDS banks ----
        {
            uint16_t *so = reinterpret_cast<uint16_t *>(s_w + ((st_last * kTileWaves + wave) * TPW) * 64);
#pragma unroll
            for (int hf = 0; hf < HALVES; ++hf) {
#pragma unroll
                for (int tt = 0; tt < TH; ++tt)
#pragma unroll
                    for (int sb = 0; sb < NS; ++sb) {
                        const floatx4 v = tot[hf * TH + tt][sb];
                        const float r4[4] = {v.x, v.y, v.z, v.w};
                        if (SWI) {
                            // lane n16 < 8 holds the gate row of feature n16 for
                            // token rows 4 kq + 0..3, lane n16 + 8 the up row: the
                            // gate lane forms rows 0 and 1 (it receives two up
                            // values), the up lane rows 2 and 3 (two gate values)
                            const bool gl = n16 < 8;
#pragma unroll
                            for (int j = 0; j < 2; ++j) {
                                const float recv = row_swap8(gl ? r4[j + 2] : r4[j]);
                                const float gate = gl ? r4[j] : recv, up = gl ? recv : r4[j + 2];
                                const int rr = sb * 16 + kq * 4 + (gl ? j : j + 2);
                                so[rr * OCOLS + ((tt ^ kq) << 3) + (n16 & 7)] =
                                    (uint16_t)bf16_pair(silu_fast(gate) * up, 0.f);
                            }
                        } else {
                            const int cs = (((tt * COLS + n16) >> 3) ^ kq) << 3 | (n16 & 7);
#pragma unroll
                            for (int i = 0; i < 4; ++i)
                                so[(sb * 16 + kq * 4 + i) * OCOLS + cs] = (uint16_t)bf16_pair(r4[i], 0.f);
                        }
                    }
                __builtin_amdgcn_wave_barrier();
                const int le = lane;
                const int part = le % LPR;
                // row le / LPR + pass * RPP has (row / 4) % 4 = (le / 16) % 4 in every pass
                static_assert(LPR == 4 && RPP % 16 == 0, "chunk swizzle per lane");
                const u32x4 *src_row =
                    reinterpret_cast<const u32x4 *>(so + (le / LPR) * OCOLS + ((part ^ ((le >> 4) & 3)) << 3));
                const uint32_t col = (uint32_t)((q.tile0 + hf * TH) * COLS + part * 8);
#pragma unroll
                for (int pass = 0; pass < CS / RPP; ++pass) {
                    const int m = pass * RPP + le / LPR;
                    const u32x4 d = src_row[pass * RPP * OCOLS / 8];
                    const uint32_t vo = m < q.nvalid ? ((uint32_t)s_crow[m] * (uint32_t)p.ldc + col) * 2u : kOutOfRange;
                    __builtin_amdgcn_raw_buffer_store_b128(d, ro, vo, 0, 0);
                }
                __builtin_amdgcn_wave_barrier();
            }
        }
        // every wave's staging reads are done (their data fed the stores):
        // the last stage is free for the next item's group 2. The wait leaves
        // only this epilogue's stores in flight (the next item's groups 0 and
        // 1 are due at its start anyway), so every load the next item's first
        // instructions use is known complete.
        wait_barrier(std::integral_constant<int, NST>());
#pragma unroll
        for (int t = 0; t < TPW; ++t)
            csc[t] = csc_n[t];
        crow = crow_n;
        src_cur = src_n1;
        src_n1 = src_n2;
        q_cur = q_nxt;
        q_nxt = qnn;
        st0 = (st0 + G) % 3;
    }
    {
        constexpr uint32_t W0 = vmcnt_imm(0);            // no copy lands after the workgroup ends
        __builtin_amdgcn_s_waitcnt(W0);
    }
}

// ---------------------------------------------------------------------------
// launch selection
// ---------------------------------------------------------------------------

long long grid_for(long long items, int wg_per_cu)
{
    const long long cap = (long long)device_cu_count() * wg_per_cu;
    long long g = items < cap ? items : cap;
    return g < 1 ? 1 : g;
}

// Workgroups of `kernel` (256 threads) one CU holds at once, per instance.
// Cached per (kernel, dynamic LDS size): the occupancy query is not free.
template <typename F>
int resident_per_cu(F kernel, size_t lds = 0)
{
    static std::mutex mu;
    static std::map<std::pair<const void *, size_t>, int> cache;
    const auto key = std::make_pair(reinterpret_cast<const void *>(kernel), lds);
    std::lock_guard<std::mutex> lock(mu);
    auto it = cache.find(key);
    if (it != cache.end())
        return it->second;
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, 256, lds) != hipSuccess || n < 1)
        n = 1;
    cache[key] = n;
    return n;
}

template <int KIND, int TPW, int NSUB, int KSEG, int RING, bool NT, int SRC = SRC_OFFSETS, int PL = 8>
hipError_t launch_stream(const GemmArgs &a, int max_rows, hipStream_t st)
{
    constexpr int CS = 16 * NSUB;
    auto kernel = gemm_stream_kernel<KIND, TPW, NSUB, KSEG, RING, NT, SRC, PL>;
    const size_t tables = SRC == SRC_OFFSETS ? sizeof(int) * (2 * (a.num_experts + 1) + 4)
                          : SRC == SRC_IDS   ? sizeof(int) * (2 * (a.num_experts + 1) + 8) +
                                                   2 * (size_t)a.T * (a.top_k + a.num_experts - a.e_routed)
                                             : sizeof(int) * (2 * kDecMaxSlots + 4 + a.num_experts);
    const size_t lds = stream_act_bytes<NSUB, KSEG>() + tables;
    const int per_cu = resident_per_cu(kernel, lds);
    // persistent grid: at most the resident slots, at most the item bound
    // (small batch: at most one item per slot and block)
    const int nblocks = (a.N >> 4) / (4 * TPW);
    const long long chunks = (SRC == SRC_ROUTE || SRC == SRC_SLOTS)
                                 ? (long long)min(a.num_experts, max_rows)
                                 : (long long)min(a.num_experts, max_rows) + max_rows / CS;
    long long grid = grid_for(chunks * nblocks, per_cu);
    if (grid >= kXcds)
        grid -= grid % kXcds;                          // whole XCD shares (see the kernel)
    hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(256), lds, st, a);
    return hipGetLastError();
}

template <int KIND, int WAVES, int NS>
hipError_t launch_tile(const GemmArgs &a, int max_rows, hipStream_t st)
{
    auto kernel = gemm_tile_kernel<KIND, WAVES, NS>;
    const size_t lds = tile_lds_bytes(WAVES, NS, a.num_experts);
    const int nblocks = (a.N >> 4) / (4 * WAVES);
    const long long chunks = (long long)min(a.num_experts, max_rows) + max_rows / (16 * NS);
    // one workgroup per CU for 8 waves, two for 4 (their LDS)
    long long grid = grid_for(chunks * nblocks, WAVES == 8 ? 1 : 2);
    if (grid >= kXcds)
        grid -= grid % kXcds;                          // whole XCD shares (see the streaming kernel)
    hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(WAVES * 64), lds, st, a);
    return hipGetLastError();
}

template <int KIND, int NWAVES>
hipError_t launch_splitk(const GemmArgs &a, int max_rows, hipStream_t st)
{
    const long long chunks = (long long)min(a.num_experts, max_rows) + max_rows / 16;
    const long long grid = grid_for(chunks * (a.N >> 4), 16 / NWAVES > 0 ? 16 / NWAVES : 1);
    hipLaunchKernelGGL((gemm_splitk_kernel<KIND, NWAVES, 4>), dim3((unsigned)grid), dim3(NWAVES * 64), 0, st, a);
    return hipGetLastError();
}

template <int KIND>
hipError_t launch_kind(const GemmArgs &a, int max_rows, int mode, int tpw, int nsub, int kseg, int ring, bool nt,
                       hipStream_t st)
{
    if (mode == 2)
        return launch_tile<KIND, 8, 4>(a, max_rows, st);
    if (mode == 3)
        return launch_tile<KIND, 4, 2>(a, max_rows, st);
    if (mode == 0) {
        switch (splitk_waves(a.K / kGroup)) {
        case 8: return launch_splitk<KIND, 8>(a, max_rows, st);
        case 4: return launch_splitk<KIND, 4>(a, max_rows, st);
        case 2: return launch_splitk<KIND, 2>(a, max_rows, st);
        default: return launch_splitk<KIND, 1>(a, max_rows, st);
        }
    }
#define MOE_STREAM(T, S, B, R)                                \
    if (tpw == T && nsub == S && kseg == B && ring == R)      \
        return nt ? launch_stream<KIND, T, S, B, R, true>(a, max_rows, st)    \
                  : launch_stream<KIND, T, S, B, R, false>(a, max_rows, st);
    MOE_STREAM(1, 1, 2, 2) MOE_STREAM(1, 1, 4, 2) MOE_STREAM(1, 1, 4, 4) MOE_STREAM(1, 1, 8, 4) MOE_STREAM(1, 2, 2, 2)
    MOE_STREAM(1, 2, 4, 2) MOE_STREAM(1, 2, 4, 4)
    MOE_STREAM(1, 4, 2, 2)
    MOE_STREAM(2, 1, 2, 2) MOE_STREAM(2, 1, 4, 2) MOE_STREAM(2, 1, 4, 4) MOE_STREAM(2, 1, 8, 4)
    MOE_STREAM(2, 2, 2, 2) MOE_STREAM(2, 2, 4, 2) MOE_STREAM(2, 2, 4, 4) MOE_STREAM(2, 4, 2, 2)
    MOE_STREAM(4, 1, 2, 2) MOE_STREAM(4, 1, 4, 2) MOE_STREAM(4, 1, 4, 4) MOE_STREAM(4, 1, 8, 4)
    MOE_STREAM(4, 2, 2, 2) MOE_STREAM(4, 2, 4, 2) MOE_STREAM(4, 2, 4, 4) MOE_STREAM(4, 4, 2, 2)
    MOE_STREAM(2, 4, 1, 2) MOE_STREAM(4, 4, 1, 2)
#undef MOE_STREAM
    // no streaming instance for this combination: the split-K kernel takes any shape
    return launch_kind<KIND>(a, max_rows, 0, tpw, nsub, kseg, ring, nt, st);
}

}  // namespace

// Streaming kernel instances (tiles per wave, subtiles, K segment, ring depth).
static bool stream_instance(int tpw, int nsub, int kseg, int ring)
{
    static const int list[][4] = {{1, 1, 2, 2}, {1, 1, 4, 2}, {1, 1, 4, 4}, {1, 1, 8, 4}, {1, 2, 2, 2}, {1, 2, 4, 2},
                                  {1, 2, 4, 4}, {1, 4, 2, 2}, {2, 1, 2, 2}, {2, 1, 4, 2}, {2, 1, 4, 4}, {2, 1, 8, 4},
                                  {2, 2, 2, 2}, {2, 2, 4, 2}, {2, 2, 4, 4}, {2, 4, 2, 2}, {4, 1, 2, 2}, {4, 1, 4, 2},
                                  {4, 1, 4, 4}, {4, 1, 8, 4}, {4, 2, 2, 2}, {4, 2, 4, 2}, {4, 2, 4, 4}, {4, 4, 2, 2},
                                  {2, 4, 1, 2}, {4, 4, 1, 2}};
    for (const auto &l : list)
        if (l[0] == tpw && l[1] == nsub && l[2] == kseg && l[3] == ring)
            return true;
    return false;
}

// Shapes the tile kernel takes: tiled codes, K/128 even, at least 4 (the
// next item's first groups are copied during groups G-3 and G-2) and at most
// 16 (one correction column per group), 512-row blocks, expert tables in the
// LDS left over, bf16 output that 32-bit buffer offsets reach.
static bool tile_fits(const GemmLaunch &g, int waves)
{
    const int G = g.K / kGroup;
    const int ldc = g.kind == MOE_GEMM_W13_SWIGLU ? g.N / 2 : g.N;
    return g.w_tiled && G % 2 == 0 && G >= 4 && G <= 16 && (g.N / 16) % (4 * waves) == 0 &&
           g.num_experts <= 256 && (g.kind == MOE_GEMM_W13_SWIGLU || !g.c_f32) &&
           (size_t)g.max_rows * (size_t)ldc * 2 < 0x80000000u;
}

static GemmArgs make_args(const GemmLaunch &g)
{
    GemmArgs a{};
    a.a = g.a;
    a.a_row_index = g.a_row_index;
    a.offsets = g.offsets;
    a.wq = g.wq;
    a.wq_sh = g.wq_sh;
    a.s_sh = g.s_sh;
    a.e_routed = g.wq_sh ? g.e_routed : g.num_experts;
    a.s = g.s;
    a.dense_rows = g.dense_rows;
    a.c = g.c;
    a.c_row_index = g.c_row_index;
    a.c_row_bytes = g.c_row_index ? (uint32_t)g.max_rows * 4u : 0u;
    a.a_row_bytes = g.a_row_index ? (uint32_t)g.max_rows * 4u : 0u;
    a.a_bytes = (uint32_t)g.a_bytes;
    a.top_k = g.top_k;
    a.num_experts = g.num_experts;
    a.K = g.K;
    a.N = g.N;
    a.c_f32 = g.c_f32 ? 1 : 0;
    a.w_tiled = g.w_tiled ? 1 : 0;
    a.half = g.N / 2;
    a.ldc = (g.kind == MOE_GEMM_W13_SWIGLU) ? g.N / 2 : g.N;
    {
        const size_t cb = (size_t)g.max_rows * (size_t)a.ldc * 2;
        a.c_bytes = cb < 0x80000000u ? (uint32_t)cb : 0u;   // 0: too large for the tile kernel
    }
    return a;
}

// The launch the grouped GEMM takes for this shape: kernel family (mode 0
// split-K, 1 streaming, 2 / 3 tile kernel) and its tiling.
LaunchChoice choose_launch(const GemmLaunch &g)
{
    // Expected rows per active expert (uniform routing estimate) picks the
    // kernel and the tile shape. Only the launch shape depends on it, never
    // the result.
    const double E = g.num_experts > 0 ? g.num_experts : 1;
    const double R = g.expected_rows > 0 ? g.expected_rows : 1;
    const double T = g.max_rows / (double)(g.top_k > 0 ? g.top_k : 1);
    const double p_slot = R / (T * E);                   // P(token routes to a given expert)
    const double active = E * (1.0 - pow(1.0 - (p_slot < 1.0 ? p_slot : 1.0), T));
    const double m = R / (active > 1.0 ? active : 1.0);
    const int G = g.K / kGroup;
    const int ntiles = g.N / 16;
    // Measured on MI355X (Qwen3-30B-A3B and EP-shard MoE shapes at 1..2048
    // tokens, dense GEMMs of 1..1024 rows):
    //  * a second 16-token subtile once experts average more than 12 rows
    //    (each expert's weights are then streamed once instead of twice);
    //  * tiles per wave: 4 (the correction MFMAs and the LDS activation
    //    reads of a subtile serve four tiles), halved while the streaming
    //    kernel would not have more than two waves per CU with two subtiles
    //    (chunks x tiles / tiles-per-wave), four with one; split-K only when
    //    even one tile per wave cannot fill the chip (one or two active
    //    experts). With one subtile, 4 tiles per wave against 2: 16 tokens
    //    27.1 vs 29.6 us (GEMM1), 64 tokens 37.9 vs 39.9 us; the EP shard at
    //    64 and 256 tokens 5-7% faster;
    //  * 4-group K segments (8 for K >= 4096); a 4-deep weight ring for
    //    K >= 4096, else 2 (at 16 and 64 tokens a 2-deep ring is 3-5% faster
    //    than a 4-deep one), and 2 with four tiles and two subtiles (a
    //    deeper ring would not fit two waves per SIMD);
    //  * prefill (2048 tokens) runs best with the two-subtile shape: four
    //    subtiles with one group per segment came out 8% slower.
    const double fill = 2.0 * device_cu_count();
    // expert loads vary around m, so a second subtile pays from m > 12; one
    // expert (a dense GEMM) has exactly m rows
    const int nsub0 = (g.num_experts == 1 ? m > 16.0 : m > 12.0) ? 2 : 1;
    const double chunks = fmax(active, R / (16.0 * nsub0));
    int nsub = nsub0;
    int tpw = 4;
    const double keep = nsub == 2 ? fill : 2.0 * fill;
    while (tpw > 1 && chunks * ntiles / tpw <= keep)
        tpw >>= 1;
    int mode = chunks * ntiles / tpw > fill ? 1 : 0;
    // at most 16 routed rows of about one row per expert (one or two decode
    // tokens of top-8): split-K, whose waves issue all their code loads
    // before the first MFMA. Measured on MI355X (Qwen3-30B-A3B layer): 1
    // token 18.3 vs 20.7 us, 2 tokens 21.9 vs 23.4 us; from 4 tokens on (32
    // rows) the streaming kernel is faster (29.6 vs 37.8 us).
    if (g.num_experts > 1 && g.max_rows <= 16 && m < 1.5)
        mode = 0;
    int kseg = 4;
    int ring = g.K >= 4096 ? 4 : 2;
    if (g.K >= 4096)
        kseg = 8;
    if (tpw == 4 && nsub == 2)
        ring = 2;
    // the tile kernel (64-row chunks, 512-row blocks, both operands through
    // LDS-DMA) once experts average about 96 rows or more, 64 for the down
    // GEMM (measured on MI355X, Qwen3-30B-A3B shapes: at 64 rows per expert
    // 7% faster for the down GEMM, 5% slower for the gate/up GEMM; at 16 rows
    // slower for both). The 4-wave variant (32-row chunks, two workgroups per
    // CU, forced with gemm_mode 3) came out within run-to-run spread of the
    // streaming kernel from 16 to 64 rows per expert and is not chosen.
    if (m >= (g.kind == MOE_GEMM_W2 ? 64.0 : 96.0) && tile_fits(g, 8))
        mode = 2;
    const moe_launch_override ov = launch_override();
    if (ov.gemm_mode >= 0)
        mode = ov.gemm_mode;
    if (ov.gemm_tiles_per_wave > 0)
        tpw = ov.gemm_tiles_per_wave;
    if (ov.gemm_subtiles > 0)
        nsub = ov.gemm_subtiles;
    if (ov.gemm_kseg > 0)
        kseg = ov.gemm_kseg;
    if (ov.gemm_ring > 0)
        ring = ov.gemm_ring;
    while (tpw > 1 && ntiles % (4 * tpw) != 0)
        tpw >>= 1;
    // LDS: 2 buffers x KSEG groups x NSUB subtiles x 4 KiB <= 64 KiB
    while (kseg > 2 && (G % kseg != 0 || 2 * kseg * nsub * 4 > 64))
        kseg >>= 1;
    if (kseg % ring != 0 && !(kseg == 1 && ring == 2))   // instantiated ring depths
        ring = 2;
    if ((mode == 2 && !tile_fits(g, 8)) || (mode == 3 && !tile_fits(g, 4)))
        mode = 1;
    if (mode == 1 && (ntiles % (4 * tpw) != 0 || G % kseg != 0 || !stream_instance(tpw, nsub, kseg, ring)))
        mode = 0;                                         // shapes the streaming tiles do not divide
    // non-temporal code loads while most experts fit one chunk (their codes
    // are then read once): routed loads vary around m, a dense GEMM has
    // exactly m rows
    bool nt = m <= (g.num_experts == 1 ? 1.0 : 0.75) * 16.0 * nsub;
    if (ov.gemm_nontemporal >= 0)
        nt = ov.gemm_nontemporal != 0;
    LaunchChoice c;
    c.mode = mode;
    c.tpw = tpw;
    c.nsub = nsub;
    c.kseg = kseg;
    c.ring = ring;
    c.nt = nt;
    return c;
}

hipError_t launch_grouped_gemm(const GemmLaunch &g, hipStream_t st)
{
    const GemmArgs a = make_args(g);
    const LaunchChoice c = choose_launch(g);
    if (g.kind == MOE_GEMM_W13_SWIGLU)
        return launch_kind<MOE_GEMM_W13_SWIGLU>(a, g.max_rows, c.mode, c.tpw, c.nsub, c.kseg, c.ring, c.nt, st);
    return launch_kind<MOE_GEMM_W2>(a, g.max_rows, c.mode, c.tpw, c.nsub, c.kseg, c.ring, c.nt, st);
}

// The layer's small-batch path on the streaming kernel: the item source is
// the slot table (SRC_ROUTE: routing inside, gate/up; SRC_SLOTS: the stored
// table, down). The tiling is choose_launch's (one 16-row subtile at these
// row counts); every streaming tiling computes the same bits. Deeper weight rings (all 16
// groups of a tile in flight) were measured on MI355X and did not pay: one
// token's gate/up kernel went from 11.5 to 12.4 us and 16 tokens' layer from
// 50.7 to 56.1 us, so the launch is latency-chained rather than short of
// bytes in flight.
hipError_t launch_decode_stream(const GemmLaunch &g, const DecodeSource &d, hipStream_t st)
{
    GemmArgs a = make_args(g);
    a.logits = d.logits;
    a.T = d.T;
    a.E_g = d.E_g;
    a.begin = d.begin;
    a.ids = d.ids;
    a.wts = d.w;
    a.pres = d.pres;
    const LaunchChoice c = choose_launch(g);
    const int tpw = c.tpw;
    const int ntiles = g.N / 16;
    if (ntiles % (4 * tpw) != 0 || g.c_f32)
        return hipErrorInvalidValue;
#define MOE_DEC_STREAM(T_, KS_, RG_)                                                                         \
    if (tpw == T_ && c.kseg == KS_ && c.ring == RG_) {                                                     \
        if (d.src == SRC_ROUTE && g.kind == MOE_GEMM_W13_SWIGLU)                                          \
            return d.E_g <= 128                                                                           \
                       ? launch_stream<MOE_GEMM_W13_SWIGLU, T_, 1, KS_, RG_, true, SRC_ROUTE, 8>(a, g.max_rows, st) \
                       : launch_stream<MOE_GEMM_W13_SWIGLU, T_, 1, KS_, RG_, true, SRC_ROUTE, 16>(a, g.max_rows, st); \
        if (d.src == SRC_SLOTS && g.kind == MOE_GEMM_W2)                                                  \
            return launch_stream<MOE_GEMM_W2, T_, 1, KS_, RG_, true, SRC_SLOTS, 8>(a, g.max_rows, st);     \
        return hipErrorInvalidValue;                                                                      \
    }
    MOE_DEC_STREAM(1, 2, 2) MOE_DEC_STREAM(1, 4, 2) MOE_DEC_STREAM(1, 4, 4) MOE_DEC_STREAM(1, 8, 4)
    MOE_DEC_STREAM(2, 2, 2) MOE_DEC_STREAM(2, 4, 2) MOE_DEC_STREAM(2, 4, 4) MOE_DEC_STREAM(2, 8, 4)
    MOE_DEC_STREAM(4, 2, 2) MOE_DEC_STREAM(4, 4, 2) MOE_DEC_STREAM(4, 4, 4) MOE_DEC_STREAM(4, 8, 4)
#undef MOE_DEC_STREAM
    return hipErrorInvalidValue;
}

// The layer's gate/up GEMM on the streaming kernel with the permutation
// built inside it from the routing ids (SRC_IDS); the GEMM is the one
// launch_grouped_gemm runs for g (same tiling, same bits), and workgroup 0
// stores the permutation's tables for the down GEMM and the finalize.
#define MOE_IDS_STREAM_LIST(X) X(4, 1, 4, 2) X(4, 2, 4, 2) X(4, 1, 8, 4) X(4, 1, 4, 4) X(4, 1, 2, 2) \
    X(4, 2, 2, 2) X(2, 1, 4, 2) X(2, 2, 4, 2) X(2, 1, 8, 4) X(2, 1, 2, 2) X(2, 2, 2, 2) X(1, 1, 2, 2)  \
    X(1, 1, 4, 2) X(1, 2, 2, 2)

static bool ids_instance(const LaunchChoice &c)
{
#define MOE_IDS_HAS(T_, S_, B_, R_) if (c.tpw == T_ && c.nsub == S_ && c.kseg == B_ && c.ring == R_) return true;
    MOE_IDS_STREAM_LIST(MOE_IDS_HAS)
#undef MOE_IDS_HAS
    return false;
}

bool gemm_ids_supported(const GemmLaunch &g, int T)
{
    if (g.kind != MOE_GEMM_W13_SWIGLU || g.c_f32 || g.num_experts > 256 || g.offsets == nullptr)
        return false;
    const LaunchChoice c = choose_launch(g);
    if (c.mode != 1 || !ids_instance(c) || g.max_rows > kIdsPerThread * 256)
        return false;
    // the bitmaps, word prefixes and local ids fit the activation buffers
    const size_t act = sizeof(u32x4) * 2 * c.kseg * c.nsub * 4 * 64;
    return ids_scratch_bytes(g.num_experts, T) <= act;
}

hipError_t launch_gemm_ids(const GemmLaunch &g, const IdsSource &src, hipStream_t st)
{
    if (!gemm_ids_supported(g, src.T))
        return hipErrorInvalidValue;
    GemmArgs a = make_args(g);
    a.a_row_index = nullptr;
    a.a_row_bytes = 0;
    a.ids = const_cast<int32_t *>(src.ids);
    a.T = src.T;
    a.begin = src.begin;
    a.cnt_out = src.counts;
    a.off_out = src.offsets;
    a.perm_out = src.perm;
    a.inv_out = src.inv_perm;
    const LaunchChoice c = choose_launch(g);
#define MOE_IDS_LAUNCH(T_, S_, B_, R_)                                                                 \
    if (c.tpw == T_ && c.nsub == S_ && c.kseg == B_ && c.ring == R_)                                 \
        return c.nt ? launch_stream<MOE_GEMM_W13_SWIGLU, T_, S_, B_, R_, true, SRC_IDS>(a, g.max_rows, st) \
                    : launch_stream<MOE_GEMM_W13_SWIGLU, T_, S_, B_, R_, false, SRC_IDS>(a, g.max_rows, st);
    MOE_IDS_STREAM_LIST(MOE_IDS_LAUNCH)
#undef MOE_IDS_LAUNCH
    return hipErrorInvalidValue;
}
#undef MOE_IDS_STREAM_LIST

// Whether launch_decode_stream has an instance for this GEMM.
bool decode_stream_supported(const GemmLaunch &g)
{
    const LaunchChoice c = choose_launch(g);
    if (c.mode != 1 || (g.N / 16) % (4 * c.tpw) != 0 || g.c_f32)
        return false;
    return (c.kseg == 2 && c.ring == 2) || (c.kseg == 4 && (c.ring == 2 || c.ring == 4)) || (c.kseg == 8 && c.ring == 4);
}

}  // namespace moe

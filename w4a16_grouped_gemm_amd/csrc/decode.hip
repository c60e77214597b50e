// decode.hip -- the layer's small-batch path (1 to 16 tokens): two or three
// launches instead of five, and no permutation.
//
// Pages: GC-MoE abstract (decode holds 1-256 tokens per rank and is dominated
// by dispatch latency and weight traffic); FlashInfer PR #7196 analysis,
// section 2 (only routed rows are computed; the MMA's token extent follows
// the routed-token count) and section 1 (the combine: fp32 multiply for the
// first slot, fp32 FMA for later slots in slot order); InfiniLM PR #500
// report, section 2.2 (the layer's steps).
//
// With at most 16 tokens every expert holds at most 16 routed rows, one
// MFMA subtile, so no permutation is needed: a workgroup that knows the
// routing can list an expert's rows itself.
//  * gate/up (decode_gate_up_kernel, or the streaming kernel with routing
//    inside): every workgroup routes all T tokens itself (the
//    logits are a few KiB), so routing costs no launch and no memory round
//    trip of its own. The "leader" of an expert is its first slot in slot
//    order; items are (leader, 16-row weight tile). An item's rows are the
//    slots routed to that expert, in token order; their SwiGLU outputs go
//    to h in slot order (row t*k + j). Workgroup 0 also writes each slot's
//    expert id, routing weight and presence (slot index, or -1 when the
//    expert is not local).
//  * down (decode_down_kernel, or the streaming kernel on the stored slot
//    table; otherwise): the same items from the stored slot
//    table; y in slot order, then the finalize kernel reads y[t*k + j].
//  * decode_down_combine_kernel (T <= 2, few h bytes per token): items are
//    (token, 16-column tile);
//    the workgroup computes the tile for each of the token's present slots
//    and combines them in slot order (multiply, then FMA), so the finalize
//    needs no launch of its own. An expert used by several of the tokens is
//    then streamed once per token (at 4 tokens of top-8 over 128 experts,
//    about 12% more down-projection bytes than once per expert).
// Every tile repeats the arithmetic of the kernel family the standalone
// grouped GEMM picks for the same shape: the split-K body of gemm_core.hpp
// with the same wave split (the kernels here), or the streaming kernel itself
// with the slot table as its item source (gemm_w4a16.hip); the combine
// repeats the finalize kernel's operations. The path is therefore
// bit-identical to the standalone entry points composed.
#include "gemm_core.hpp"
#include "route_core.hpp"

#include <map>
#include <mutex>
#include <utility>

namespace moe {

namespace {

struct DecodeArgs {
    int T, k, E_g, begin, E_loc;
    const float *logits;                // [T][E_g] (gate/up kernel)
    int32_t *ids;                       // [T*k] global expert id of each slot
    float *w;                           // [T*k] routing weight
    int32_t *pres;                      // [T*k] slot index if its expert is local, else -1
    const uint16_t *a;                  // gate/up: x [T][K]; down: h [T*k][K]
    uint32_t a_bytes;
    const uint8_t *wq;                  // codes of the local experts
    const uint16_t *s;                  // scales
    int K, N, w_tiled;
    uint16_t *c;                        // gate/up: h [T*k][N/2]; down: y [T*k][N]; combine: out [T][N]
};

// Weight row of lane n16 in tile `tile` (gate/up: gate rows 8t.., then the
// matching up rows; down: 16t + n16) and the lane offset of its codes.
template <int KIND>
__device__ __forceinline__ uint32_t dec_row(const DecodeArgs &p, int tile, int n16)
{
    if (KIND == MOE_GEMM_W13_SWIGLU)
        return (uint32_t)(n16 < 8 ? tile * 8 + n16 : p.N / 2 + tile * 8 + (n16 - 8));
    return (uint32_t)(tile * 16 + n16);
}

__device__ __forceinline__ uint32_t dec_code_offset(const DecodeArgs &p, int tile, uint32_t row, int G, int lane)
{
    if (p.w_tiled)
        return (uint32_t)((tile >> 3) * G * 8 + (tile & 7)) * 1024u + (uint32_t)lane * 16u;
    return row * (uint32_t)(p.K >> 1) + (uint32_t)(lane >> 4) * 16u;
}

// One expert-major item: expert e (leader slot `lead`), 16-row tile `tile`.
// Rows are the slots of expert e in slot order; row r reads activation row
// a_row(slot) and its result goes to output row `slot`.
template <int KIND, int NW, bool A_BY_TOKEN>
__device__ __forceinline__ void expert_item(const DecodeArgs &p, const int *s_loc, floatx4 (*s_red)[64], int e,
                                            int tile, int S)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, n16 = lane & 15, kq = lane >> 4;
    const int G = p.K / kGroup;
    int g0, g1;
    splitk_groups(wave, G, NW, g0, g1);
    // the expert's slots: bits of (m0, m1) over slots 0..127
    const uint64_t m0 = __ballot(lane < S && s_loc[lane] == e);
    const uint64_t m1 = __ballot(64 + lane < S && s_loc[64 + lane] == e);
    const int nrows = __popcll(m0) + __popcll(m1);
    const int my_slot = nth_slot(m0, m1, n16);         // activation row of lane n16
    const uint32_t wbytes = (uint32_t)p.N * (uint32_t)(p.K >> 1);
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(p.wq + (size_t)e * wbytes, wbytes);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.s + (size_t)e * p.N * G, (uint32_t)p.N * G * 2);
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.a, p.a_bytes);
    const uint32_t row = dec_row<KIND>(p, tile, n16);
    const uint32_t voff_w = dec_code_offset(p, tile, row, G, lane);
    const uint32_t voff_s = row * (uint32_t)G * 2;
    uint32_t voff_x = kOutOfRange;
    if (my_slot >= 0) {
        const uint32_t src = A_BY_TOKEN ? (uint32_t)(my_slot / p.k) : (uint32_t)my_slot;
        voff_x = src * (uint32_t)p.K * 2 + kq * 64;
    }
    const floatx4 tot = splitk_wave_sum<4>(rw, voff_w, p.w_tiled ? 8192u : 64u, rs, voff_s, ra, voff_x, g0, g1,
                                           p.w_tiled != 0);
    const floatx4 sum = splitk_reduce<NW>(tot, s_red, wave, lane);
    if (wave != 0)
        return;
    const float r[4] = {sum.x, sum.y, sum.z, sum.w};
    int orow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        orow[i] = __shfl(my_slot, kq * 4 + i, 64);       // output row of result row 4kq + i
    if (KIND == MOE_GEMM_W13_SWIGLU) {
        float u[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            u[i] = __shfl_xor(r[i], 8, 64);               // partner lane holds the up row
        if (n16 < 8) {
            const int ldc = p.N / 2;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (kq * 4 + i < nrows)
                    p.c[(size_t)orow[i] * ldc + tile * 8 + n16] = (uint16_t)f32_to_bf16_rne(silu(r[i]) * u[i]);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (kq * 4 + i < nrows)
                p.c[(size_t)orow[i] * p.N + tile * 16 + n16] = (uint16_t)f32_to_bf16_rne(r[i]);
    }
}

// Gate/up with routing inside: every workgroup routes all tokens (TL lanes
// per token, PL logits per lane, E_g <= TL * PL), builds the slot table and
// the leaders, then runs its share of the (leader, tile) items. With at most
// one token per wave a whole wave routes each token (TL = 64): the k rounds
// of the selection are the routing's serial part, and 64 lanes of PL = 2
// logits (128 experts) take about half the instructions per round of 16
// lanes of 8. The selection and the weights are those of the 16-lane shape
// bit for bit (the same comparisons; the slot weights are formed in lanes
// 0..k-1, one DPP row, as there).
template <int NW, int TL, int PL>
__global__ __launch_bounds__(NW * 64) void decode_gate_up_kernel(DecodeArgs p)
{
    __shared__ int s_loc[kDecMaxSlots];
    __shared__ int s_first[kMaxExperts];
    __shared__ int s_lead[kDecMaxSlots];
    __shared__ int s_nlead;
    __shared__ floatx4 s_red[NW][64];
    constexpr int TPWV = 64 / TL;                      // tokens per wave and pass
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, q = lane % TL;
    const int S = p.T * p.k;
    for (int e = tid; e < p.E_loc; e += NW * 64)
        s_first[e] = kDecMaxSlots;
    for (int t0 = wave * TPWV; t0 < p.T; t0 += NW * TPWV) {
        const int t = t0 + lane / TL;
        if (t < p.T) {
            int eg;
            float wt;
            route_token<TL, PL>(p.logits + (size_t)t * p.E_g, p.E_g, p.k, q, eg, wt);
            if (q < p.k) {
                const int s = t * p.k + q;
                const int le = eg - p.begin;
                const int loc = (le >= 0 && le < p.E_loc) ? le : -1;
                s_loc[s] = loc;
                if (blockIdx.x == 0) {
                    p.ids[s] = eg;
                    p.w[s] = wt;
                    p.pres[s] = loc >= 0 ? s : -1;
                }
            }
        }
    }
    __syncthreads();
    build_leaders<NW * 64>(S, p.E_loc, s_loc, s_first, s_lead, &s_nlead);
    const int ntiles = p.N >> 4;
    const int items = s_nlead * ntiles;
    for (int item = blockIdx.x; item < items; item += gridDim.x) {
        const int lead = s_lead[item / ntiles];
        expert_item<MOE_GEMM_W13_SWIGLU, NW, true>(p, s_loc, s_red, uniform(s_loc[lead]), item % ntiles, S);
    }
}

// Down projection, expert-major, from the stored slot table; y in slot order.
template <int NW>
__global__ __launch_bounds__(NW * 64) void decode_down_kernel(DecodeArgs p)
{
    __shared__ int s_loc[kDecMaxSlots];
    __shared__ int s_first[kMaxExperts];
    __shared__ int s_lead[kDecMaxSlots];
    __shared__ int s_nlead;
    __shared__ floatx4 s_red[NW][64];
    const int tid = threadIdx.x;
    const int S = p.T * p.k;
    for (int e = tid; e < p.E_loc; e += NW * 64)
        s_first[e] = kDecMaxSlots;
    for (int s = tid; s < S; s += NW * 64)
        s_loc[s] = p.pres[s] >= 0 ? p.ids[s] - p.begin : -1;
    __syncthreads();
    build_leaders<NW * 64>(S, p.E_loc, s_loc, s_first, s_lead, &s_nlead);
    const int ntiles = p.N >> 4;
    const int items = s_nlead * ntiles;
    for (int item = blockIdx.x; item < items; item += gridDim.x) {
        const int lead = s_lead[item / ntiles];
        expert_item<MOE_GEMM_W2, NW, false>(p, s_loc, s_red, uniform(s_loc[lead]), item % ntiles, S);
    }
}

// Down projection and combine, token-major. Item = (token t, 16-column tile).
// The tile of each of the token's present slots is computed with the
// arithmetic of the standalone down GEMM's kernel family: KS waves split K
// as the split-K kernel does (KS = 1: one wave sums every group in order,
// which is also the streaming kernel's per-element sum). SP wave groups take
// slots j = sp + u SP (u < SPW), so k <= SP * SPW. The token's h rows are
// staged in LDS (k * K bf16); each wave prefetches the codes and scales of
// its slots (at most GMAX groups each) before computing any. Partial sums of
// result row 0 go to LDS; wave 0 reduces them in wave order, rounds y to bf16
// and combines the present slots in slot order, as the finalize kernel does.
// The combine kernel re-stages the token's h rows for every 16-column tile,
// so it pays only while those rows are few: measured on MI355X it matches
// the down GEMM + finalize at 1-2 Qwen3-30B-A3B tokens (12 KiB of rows) and
// loses from 4 tokens, and on the EP shard (32 KiB of rows) already at 1.
constexpr int kCombineMaxHBytes = 64 * 1024;            // k * K * 2 bytes of staged h rows (LDS)
constexpr int kCombineAutoHBytes = 16 * 1024;           // the automatic choice's limits
constexpr int kCombineAutoTokens = 2;

template <int KS, int SP, int SPW, int GMAX>
__global__ __launch_bounds__(KS * SP * 64) void decode_down_combine_kernel(DecodeArgs p)
{
    constexpr int NW = KS * SP;
    // h pieces (16 bytes) per thread loaded in one batch: the automatic
    // choice's h rows (kCombineAutoHBytes) in one pass
    constexpr int CPT = (kCombineAutoHBytes / 16) / (NW * 64) < 1 ? 1
                        : (kCombineAutoHBytes / 16) / (NW * 64) > 8 ? 8 : (kCombineAutoHBytes / 16) / (NW * 64);
    extern __shared__ __align__(16) unsigned char s_dyn[];
    uint16_t *s_h = reinterpret_cast<uint16_t *>(s_dyn);                     // [k][K]
    __shared__ float s_part[kMaxTopK][KS][16];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, n16 = lane & 15, kq = lane >> 4;
    const int sp = wave / KS, ks = wave % KS;
    const int k = p.k, K = p.K, G = K / kGroup;
    int g0, g1;
    splitk_groups(ks, G, KS, g0, g1);
    const int ntiles = p.N >> 4;
    const uint32_t wbytes = (uint32_t)p.N * (uint32_t)(K >> 1);
    const uint32_t gstride = p.w_tiled ? 8192u : 64u;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.a, p.a_bytes);
    const int chunks = k * K / 8;                         // 16-byte pieces of the token's h rows
    for (int item = blockIdx.x; item < p.T * ntiles; item += gridDim.x) {
        const int t = item / ntiles, tile = item % ntiles;
        // slot table of token t: lane j < k holds slot j
        const int js = min(lane, k - 1);
        const int pres_l = p.pres[t * k + js];
        const int id_l = p.ids[t * k + js];
        const float w_l = p.w[t * k + js];
        // the token's k h rows: the first CPT pieces of each thread go out
        // with the slot-table loads above (no dependence on them: rows of
        // absent slots are loaded too and never read) and land in LDS after
        // the weight loads below have been issued, so the whole item costs
        // one round trip after the slot table
        const uint32_t hoff = (uint32_t)t * (uint32_t)k * (uint32_t)K * 2u;
        u32x4 hv[CPT];
#pragma unroll
        for (int u = 0; u < CPT; ++u) {
            const int c = tid + u * NW * 64;
            hv[u] = bload16(ra, c < chunks ? hoff + (uint32_t)c * 16u : kOutOfRange, 0);
        }
        // this wave's slots: codes and scales of groups g0..g1 (absent: zeros, no traffic)
        u32x4 wv[SPW][GMAX];
        uint32_t sc[SPW][GMAX];
        int jj[SPW];
        bool present[SPW];
        const uint32_t row = (uint32_t)(tile * 16 + n16);
        const uint32_t voff_w = p.w_tiled ? (uint32_t)((tile >> 3) * G * 8 + (tile & 7)) * 1024u + (uint32_t)lane * 16u
                                          : row * (uint32_t)(K >> 1) + (uint32_t)(lane >> 4) * 16u;
        const uint32_t voff_s = row * (uint32_t)G * 2;
#pragma unroll
        for (int u = 0; u < SPW; ++u) {
            const int j = sp + u * SP;
            jj[u] = j;
            const int pj = __shfl(pres_l, min(j, k - 1), 64);
            present[u] = j < k && pj >= 0;
            const int e = present[u] ? __shfl(id_l, min(j, k - 1), 64) - p.begin : 0;
            const __amdgpu_buffer_rsrc_t rw = make_rsrc(p.wq + (size_t)uniform(e) * wbytes, present[u] ? wbytes : 0u);
            const __amdgpu_buffer_rsrc_t rs =
                make_rsrc(p.s + (size_t)uniform(e) * p.N * G, present[u] ? (uint32_t)p.N * G * 2 : 0u);
#pragma unroll
            for (int q = 0; q < GMAX; ++q) {
                const int g = g0 + q;
                const uint32_t oor = g < g1 ? 0u : kOutOfRange;
                wv[u][q] = bload16_codes<true>(rw, voff_w | oor, (uint32_t)(g < g1 ? g : 0) * gstride);
                sc[u][q] = bload_scale(rs, voff_s | oor, (uint32_t)(g < g1 ? g : 0) * 2u);
            }
        }
#pragma unroll
        for (int u = 0; u < CPT; ++u) {
            const int c = tid + u * NW * 64;
            if (c < chunks)
                *reinterpret_cast<u32x4 *>(s_h + (size_t)c * 8) = hv[u];
        }
        for (int c = tid + CPT * NW * 64; c < chunks; c += NW * 64)   // rows past the batch (large k * K)
            *reinterpret_cast<u32x4 *>(s_h + (size_t)c * 8) = bload16(ra, hoff + (uint32_t)c * 16u, 0);
        __syncthreads();                                  // h rows staged
#pragma unroll
        for (int u = 0; u < SPW; ++u) {
            if (!uniform(present[u]))
                continue;
            floatx4 tot = {0.f, 0.f, 0.f, 0.f};
            const uint16_t *hrow = s_h + (size_t)jj[u] * K;
#pragma unroll
            for (int q = 0; q < GMAX; ++q) {
                const int g = g0 + q;
                if (g < g1) {
                    u32x4 a[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const u32x4 v = *reinterpret_cast<const u32x4 *>(hrow + g * kGroup + kq * 32 + i * 8);
                        const u32x4 z = {0u, 0u, 0u, 0u};
                        a[i] = n16 == 0 ? v : z;              // row 0 only: the token's h row
                    }
                    // a branch on the layout, not a select (tiled codes: no permutation)
                    if (p.w_tiled) {
                        splitk_group(a, wv[u][q], sc[u][q], tot);
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            a[i] = permute_act(a[i]);
                        splitk_group(a, wv[u][q], sc[u][q], tot);
                    }
                }
            }
            if (kq == 0)
                s_part[jj[u]][ks][n16] = tot.x;
        }
        __syncthreads();
        if (wave == 0 && lane < 16) {
            float acc = 0.0f;
            bool first = true;
            for (int j = 0; j < k; ++j) {
                const int pj = __shfl(pres_l, j, 16);
                const float wj = __shfl(w_l, j, 16);
                if (pj < 0)
                    continue;
                float y = s_part[j][0][n16];
#pragma unroll
                for (int q = 1; q < KS; ++q)
                    y += s_part[j][q][n16];
                const float v = bf16_to_f32(f32_to_bf16_rne(y));
                acc = first ? __fmul_rn(v, wj) : __fmaf_rn(v, wj, acc);
                first = false;
            }
            p.c[(size_t)t * p.N + tile * 16 + n16] = (uint16_t)f32_to_bf16_rne(acc);
        }
        __syncthreads();                                  // LDS free for the next item
    }
}

// Persistent grid: the workgroups one launch keeps resident (occupancy of
// the kernel at this LDS size, cached), capped by the item bound.
long long resident_grid(const void *kernel, int threads, size_t lds, long long items)
{
    static std::mutex mu;
    static std::map<std::pair<const void *, size_t>, int> cache;
    int per_cu = 0;
    {
        std::lock_guard<std::mutex> lock(mu);
        const auto key = std::make_pair(kernel, lds);
        auto it = cache.find(key);
        if (it != cache.end()) {
            per_cu = it->second;
        } else {
            if (lds > 48 * 1024)
                (void)hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, lds) != hipSuccess ||
                per_cu < 1)
                per_cu = 1;
            cache[key] = per_cu;
        }
    }
    long long cap = (long long)device_cu_count() * per_cu;
    long long g = items < cap ? items : cap;
    return g < 1 ? 1 : g;
}

}  // namespace

// Kernel family of the layer's standalone gate/up and down GEMMs at this
// shape: the small-batch path repeats that family's arithmetic (split-K: the
// split-K body with the same wave split; streaming: the streaming kernel with
// the slot-table item source), so the layer equals the GEMMs composed.
static int gemm_family(const moe_shape &sh, moe_gemm_kind kind)
{
    return choose_launch(layer_gemm_args(sh, kind)).mode;
}

// The combine kernel's shape for this layer: waves splitting K (the down
// GEMM's split-K wave count, 1 for the streaming family), slot groups, slots
// per wave, and the most groups a wave holds.
struct CombineShape {
    int KS, SP, SPW, GMAX;
};

static CombineShape combine_shape(const moe_shape &sh)
{
    const int G = sh.inter / kGroup;
    CombineShape c{};
    c.KS = gemm_family(sh, MOE_GEMM_W2) == 0 ? splitk_waves(G) : 1;
    c.SPW = c.KS == 1 ? 1 : 2;
    c.GMAX = c.KS == 1 ? 16 : 4;
    const int need = (sh.top_k + c.SPW - 1) / c.SPW;
    c.SP = need <= 1 ? 1 : need <= 2 ? 2 : need <= 4 ? 4 : need <= 8 ? 8 : 16;
    return c;
}

bool decode_path_fits(const moe_shape &sh, int nsh)
{
    const moe_launch_override ov = launch_override();
    const int max_t = ov.decode_max_tokens >= 0 ? ov.decode_max_tokens : 16;
    if (!(nsh == 0 && sh.num_tokens <= max_t && sh.num_tokens * sh.top_k <= kDecMaxSlots && sh.num_experts <= 256))
        return false;
    const GemmLaunch g1 = layer_gemm_args(sh, MOE_GEMM_W13_SWIGLU), g2 = layer_gemm_args(sh, MOE_GEMM_W2);
    const int f1 = choose_launch(g1).mode, f2 = choose_launch(g2).mode;
    if (f1 > 1 || f2 > 1)
        return false;                                     // a tile-kernel shape: the general path
    if (f1 == 1 && !decode_stream_supported(g1))
        return false;
    return decode_combine_fits(sh) || f2 == 0 || decode_stream_supported(g2);
}

bool decode_combine_fits(const moe_shape &sh)
{
    const moe_launch_override ov = launch_override();
    const bool forced = ov.decode_combine_max_tokens >= 0;
    const int max_t = forced ? ov.decode_combine_max_tokens : kCombineAutoTokens;
    const size_t max_h = forced ? kCombineMaxHBytes : kCombineAutoHBytes;
    const int G = sh.inter / kGroup;
    const CombineShape c = combine_shape(sh);
    return sh.num_tokens <= max_t && gemm_family(sh, MOE_GEMM_W2) <= 1 && (G + c.KS - 1) / c.KS <= c.GMAX &&
           c.KS * c.SP <= 16 && (size_t)sh.top_k * sh.inter * 2 <= max_h;
}

hipError_t launch_decode_gate_up(const moe_shape &sh, const float *logits, const uint16_t *x, const uint8_t *w13,
                                 const uint16_t *s13, int32_t *ids, float *w, int32_t *pres, uint16_t *h,
                                 hipStream_t st)
{
    GemmLaunch g = layer_gemm_args(sh, MOE_GEMM_W13_SWIGLU);
    if (choose_launch(g).mode == 1) {
        g.a = x;
        g.a_bytes = (size_t)sh.num_tokens * sh.hidden * 2;
        g.wq = w13;
        g.s = s13;
        g.c = h;
        g.c_f32 = false;
        const DecodeSource d{1, logits, sh.num_tokens, sh.num_experts, sh.expert_begin, ids, w, pres};
        return launch_decode_stream(g, d, st);
    }
    DecodeArgs p{};
    p.T = sh.num_tokens;
    p.k = sh.top_k;
    p.E_g = sh.num_experts;
    p.begin = sh.expert_begin;
    p.E_loc = sh.num_local_experts;
    p.logits = logits;
    p.ids = ids;
    p.w = w;
    p.pres = pres;
    p.a = x;
    p.a_bytes = (uint32_t)((size_t)sh.num_tokens * sh.hidden * 2);
    p.wq = w13;
    p.s = s13;
    p.K = sh.hidden;
    p.N = 2 * sh.inter;
    p.w_tiled = sh.weight_layout == MOE_WEIGHTS_TILED;
    p.c = h;
    const int G = p.K / kGroup;
    const long long items = (long long)sh.num_tokens * sh.top_k * (p.N / 16);
    auto go = [&](auto kernel, int nw) {
        const long long grid = resident_grid(reinterpret_cast<const void *>(kernel), nw * 64, 0, items);
        hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(nw * 64), 0, st, p);
    };
    const int E = sh.num_experts;
    // a wave per token while every wave routes at most one (see the kernel)
#define MOE_DEC_GU(NW)                                                                     \
    if (sh.num_tokens <= NW) {                                                             \
        if (E <= 64)                                                                       \
            go(decode_gate_up_kernel<NW, 64, 1>, NW);                                      \
        else if (E <= 128)                                                                 \
            go(decode_gate_up_kernel<NW, 64, 2>, NW);                                      \
        else                                                                               \
            go(decode_gate_up_kernel<NW, 64, 4>, NW);                                      \
    } else if (E <= 64)                                                                    \
        go(decode_gate_up_kernel<NW, 16, 4>, NW);                                          \
    else if (E <= 128)                                                                     \
        go(decode_gate_up_kernel<NW, 16, 8>, NW);                                          \
    else                                                                                   \
        go(decode_gate_up_kernel<NW, 16, 16>, NW);
    switch (splitk_waves(G)) {
    case 8: MOE_DEC_GU(8) break;
    case 4: MOE_DEC_GU(4) break;
    case 2: MOE_DEC_GU(2) break;
    default: MOE_DEC_GU(1) break;
    }
#undef MOE_DEC_GU
    return hipGetLastError();
}

static DecodeArgs down_args(const moe_shape &sh, const int32_t *ids, const float *w, const int32_t *pres,
                            const uint16_t *h, const uint8_t *w2, const uint16_t *s2, uint16_t *c)
{
    DecodeArgs p{};
    p.T = sh.num_tokens;
    p.k = sh.top_k;
    p.E_g = sh.num_experts;
    p.begin = sh.expert_begin;
    p.E_loc = sh.num_local_experts;
    p.ids = const_cast<int32_t *>(ids);
    p.w = const_cast<float *>(w);
    p.pres = const_cast<int32_t *>(pres);
    p.a = h;
    p.a_bytes = (uint32_t)((size_t)sh.num_tokens * sh.top_k * sh.inter * 2);
    p.wq = w2;
    p.s = s2;
    p.K = sh.inter;
    p.N = sh.hidden;
    p.w_tiled = sh.weight_layout == MOE_WEIGHTS_TILED;
    p.c = c;
    return p;
}

hipError_t launch_decode_down(const moe_shape &sh, const int32_t *ids, const int32_t *pres, const uint16_t *h,
                              const uint8_t *w2, const uint16_t *s2, uint16_t *y, hipStream_t st)
{
    GemmLaunch g = layer_gemm_args(sh, MOE_GEMM_W2);
    if (choose_launch(g).mode == 1) {
        g.a = h;
        g.a_bytes = (size_t)sh.num_tokens * sh.top_k * sh.inter * 2;
        g.wq = w2;
        g.s = s2;
        g.c = y;
        g.c_f32 = false;
        const DecodeSource d{2, nullptr, sh.num_tokens, sh.num_experts, sh.expert_begin,
                             const_cast<int32_t *>(ids), nullptr, const_cast<int32_t *>(pres)};
        return launch_decode_stream(g, d, st);
    }
    const DecodeArgs p = down_args(sh, ids, nullptr, pres, h, w2, s2, y);
    const long long items = (long long)sh.num_tokens * sh.top_k * (p.N / 16);
    auto go = [&](auto kernel, int nw) {
        const long long grid = resident_grid(reinterpret_cast<const void *>(kernel), nw * 64, 0, items);
        hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(nw * 64), 0, st, p);
    };
    switch (splitk_waves(p.K / kGroup)) {
    case 8: go(decode_down_kernel<8>, 8); break;
    case 4: go(decode_down_kernel<4>, 4); break;
    case 2: go(decode_down_kernel<2>, 2); break;
    default: go(decode_down_kernel<1>, 1); break;
    }
    return hipGetLastError();
}

hipError_t launch_decode_down_combine(const moe_shape &sh, const int32_t *ids, const float *w, const int32_t *pres,
                                      const uint16_t *h, const uint8_t *w2, const uint16_t *s2, uint16_t *out,
                                      hipStream_t st)
{
    const DecodeArgs p = down_args(sh, ids, w, pres, h, w2, s2, out);
    const CombineShape c = combine_shape(sh);
    const size_t lds = (size_t)sh.top_k * p.K * 2;
    const long long items = (long long)sh.num_tokens * (p.N / 16);
    auto go = [&](auto kernel) {
        const int threads = c.KS * c.SP * 64;
        const long long grid = resident_grid(reinterpret_cast<const void *>(kernel), threads, lds, items);
        hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(threads), lds, st, p);
    };
#define MOE_DEC_DC(KS_, SP_, SPW_, GM_)                                                 \
    if (c.KS == KS_ && c.SP == SP_ && c.SPW == SPW_ && c.GMAX == GM_) {                  \
        go(decode_down_combine_kernel<KS_, SP_, SPW_, GM_>);                           \
        return hipGetLastError();                                                      \
    }
    MOE_DEC_DC(1, 1, 1, 16) MOE_DEC_DC(1, 2, 1, 16) MOE_DEC_DC(1, 4, 1, 16) MOE_DEC_DC(1, 8, 1, 16)
    MOE_DEC_DC(1, 16, 1, 16)
    MOE_DEC_DC(2, 1, 2, 4) MOE_DEC_DC(2, 2, 2, 4) MOE_DEC_DC(2, 4, 2, 4) MOE_DEC_DC(2, 8, 2, 4)
    MOE_DEC_DC(4, 1, 2, 4) MOE_DEC_DC(4, 2, 2, 4) MOE_DEC_DC(4, 4, 2, 4)
    MOE_DEC_DC(8, 1, 2, 4) MOE_DEC_DC(8, 2, 2, 4)
#undef MOE_DEC_DC
    return hipErrorInvalidValue;                          // decode_combine_fits() rules this out
}

}  // namespace moe

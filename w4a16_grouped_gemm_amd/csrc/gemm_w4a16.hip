// gemm_w4a16.hip -- grouped GEMM over expert slabs, int4 group-scaled weights
// x bf16 activations, fp32 accumulation on gfx950 MFMA.
//
// Method (pages): InfiniLM PR #500 report, section 2.2 (one grouped GEMM
// covers every expert slab given the group sizes; gate/up, SwiGLU, down);
// FlashInfer PR #7196 analysis, section 2 (the MMA N extent follows the
// routed-token count at run time, inactive subtiles are skipped;
// activations sit in operand B of an operand-swapped MMA); GC-MoE abstract
// (4-bit weights decoded in registers and fed straight to the matrix unit;
// decode is bound by weight traffic); Cloudflare "Unweight" post, section on
// the reconstructive matmul (weights are reconstructed on chip and never
// written back to HBM).
//
// gfx950 design (ours):
//  * MFMA v_mfma_f32_16x16x32_bf16. Operand A = 16 routed tokens of one
//    expert (a 16-token N-subtile of the expert's rows), operand B = 16 weight
//    rows. Lane l supplies token / weight row l%16 and one 8-element K slice
//    chosen by l/16; the result lane holds 4 tokens x 1 weight row, so each
//    lane needs exactly one scale per 128-wide group: the scale of its own row.
//  * Weights stream HBM -> VGPR, 16 bytes per lane per group (= 32 int4 of one
//    row), no LDS: in decode nothing is reused. Within a lane the 32 codes of
//    a group feed 4 MFMAs (K = 4 x 8 per lane x 4 lane slices = 128).
//  * Unpack is one bit-op per pair of codes: (w ^ 0x8888) & 0x000F000F |
//    0x43004300 turns two nibbles into the bf16 values 128 + (q + 8), which are
//    exact. The K order inside each 8-code dword comes out as
//    (0,4,1,5,2,6,3,7); the activation fragment is permuted the same way
//    (any common K permutation leaves the dot product unchanged).
//  * The +136 offset is removed inside the matrix unit: a second MFMA with a
//    constant -136 operand accumulates -136 * sum(x) into the same chain, so
//    the chain holds sum(x * q) exactly up to fp32 rounding (exactly, for
//    integer-valued activations). The row's fp32 scale is then applied once
//    per group: total += s * chain. Codes are never rounded.
//  * K is split over the waves of a workgroup (contiguous group ranges), the
//    partial sums are reduced through LDS in wave order (deterministic), then
//    the epilogue applies SwiGLU (gate rows 0..7 and up rows 8..15 of the
//    same 16-row tile, i.e. 8 features) or stores the plain result.
//  * Work items = (expert chunk of up to 16*NSUB rows, weight-row tile). The
//    item list is derived on the device from `offsets` by every workgroup of
//    a persistent grid, so the grid never depends on the counts and the host
//    never synchronises. Subtiles past the chunk's valid rows are skipped
//    (runtime N); rows past the last valid token are neither read nor written.
#include "common.hpp"

namespace moe {

namespace {

constexpr uint32_t kMagic = 0x43004300u;   // bf16 pair (128, 128)
constexpr uint32_t kNeg136 = 0xC308C308u;  // bf16 pair (-136, -136)

struct GemmArgs {
    const uint16_t *a;
    const int32_t *a_row_index;
    const int32_t *offsets;
    const uint8_t *wq;
    const uint16_t *s;
    void *c;
    int top_k;
    int num_experts;
    int K;
    int N;          // weight rows per expert
    int ldc;        // output row stride (elements)
    int row_tiles;  // 16-row weight tiles per expert
    int half;       // SwiGLU: row offset of the up projection (= I)
    int c_f32;
};

// Two nibbles per 16-bit half -> four bf16 pairs holding 136 + q, K order
// (0,4,1,5,2,6,3,7) within the dword.
__device__ __forceinline__ bf16x8 unpack8(uint32_t w)
{
    const uint32_t t = w ^ 0x88888888u;
    u32x4 o;
    o.x = (t & 0x000F000Fu) | kMagic;
    o.y = ((t >> 4) & 0x000F000Fu) | kMagic;
    o.z = ((t >> 8) & 0x000F000Fu) | kMagic;
    o.w = ((t >> 12) & 0x000F000Fu) | kMagic;
    return __builtin_bit_cast(bf16x8, o);
}

// Eight consecutive bf16 activations -> the same (0,4,1,5,2,6,3,7) order.
__device__ __forceinline__ bf16x8 permute_act(u32x4 d)
{
    u32x4 o;
    o.x = __builtin_amdgcn_perm(d.z, d.x, 0x05040100u);
    o.y = __builtin_amdgcn_perm(d.z, d.x, 0x07060302u);
    o.z = __builtin_amdgcn_perm(d.w, d.y, 0x05040100u);
    o.w = __builtin_amdgcn_perm(d.w, d.y, 0x07060302u);
    return __builtin_bit_cast(bf16x8, o);
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + expf(-g)); }

template <int KIND, int NWAVES, int NSUB, int GB>
__global__ __launch_bounds__(NWAVES * 64) void gemm_w4a16_kernel(GemmArgs p)
{
    constexpr int CS = 16 * NSUB;                 // rows per chunk
    __shared__ int s_prefix[kMaxExperts + 1];     // chunk prefix per expert
    __shared__ int s_wtot[NWAVES];
    __shared__ float s_red[NWAVES][CS][17];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int E = p.num_experts;

    // ---- chunk prefix over experts (device-side work list) ----
    {
        int carry = 0;
        for (int base = 0; base < E; base += NWAVES * 64) {
            const int e = base + tid;
            int v = 0;
            if (e < E) {
                const int cnt = p.offsets[e + 1] - p.offsets[e];
                v = (cnt + CS - 1) / CS;
            }
            int wt;
            const int ex = wave_exclusive_scan(v, wt);
            if (lane == 0)
                s_wtot[wave] = wt;
            __syncthreads();
            int wbase = 0, all = 0;
#pragma unroll
            for (int w = 0; w < NWAVES; ++w) {
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
    const int total_items = s_prefix[E] * p.row_tiles;
    const int G = p.K / kGroup;
    const int g0 = wave * G / NWAVES;
    const int g1 = (wave + 1) * G / NWAVES;
    const int n16 = lane & 15;
    const int kq = lane >> 4;
    const u32x4 neg136v = {kNeg136, kNeg136, kNeg136, kNeg136};
    const bf16x8 neg136 = __builtin_bit_cast(bf16x8, neg136v);

    for (int item = blockIdx.x; item < total_items; item += gridDim.x) {
        const int chunk = item / p.row_tiles;
        const int tile = item - chunk * p.row_tiles;
        // expert owning this chunk: last e with s_prefix[e] <= chunk
        int lo = 0, hi = E - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_prefix[mid] <= chunk)
                lo = mid;
            else
                hi = mid - 1;
        }
        const int e = lo;
        const int row0 = p.offsets[e] + (chunk - s_prefix[e]) * CS;
        const int nvalid = min(CS, p.offsets[e + 1] - row0);

        // this lane's weight row
        int wrow;
        if (KIND == MOE_GEMM_W13_SWIGLU)
            wrow = (n16 < 8) ? tile * 8 + n16 : p.half + tile * 8 + (n16 - 8);
        else
            wrow = tile * 16 + n16;
        const size_t wrow_index = (size_t)e * p.N + wrow;
        const uint8_t *wptr = p.wq + wrow_index * (size_t)(p.K >> 1) + kq * 16;
        const uint16_t *sptr = p.s + wrow_index * (size_t)G;

        // this lane's activation rows (one per subtile)
        const uint16_t *aptr[NSUB];
        bool aval[NSUB];
#pragma unroll
        for (int sb = 0; sb < NSUB; ++sb) {
            const int m = sb * 16 + n16;
            aval[sb] = m < nvalid;
            size_t src = 0;
            if (aval[sb]) {
                const int r = row0 + m;
                src = p.a_row_index ? (size_t)(p.a_row_index[r] / p.top_k) : (size_t)r;
            }
            aptr[sb] = p.a + src * (size_t)p.K + kq * 32;
        }

        floatx4 tot[NSUB];
#pragma unroll
        for (int sb = 0; sb < NSUB; ++sb)
            tot[sb] = floatx4{0.f, 0.f, 0.f, 0.f};

        for (int gb = g0; gb < g1; gb += GB) {
            u32x4 wv[GB];
            float sc[GB];
#pragma unroll
            for (int j = 0; j < GB; ++j) {
                if (gb + j < g1) {
                    wv[j] = *reinterpret_cast<const u32x4 *>(wptr + (size_t)(gb + j) * 64);
                    sc[j] = bf16_to_f32(sptr[gb + j]);
                }
            }
#pragma unroll
            for (int j = 0; j < GB; ++j) {
                if (gb + j >= g1)
                    break;
                const int g = gb + j;
                const bf16x8 wf0 = unpack8(wv[j].x);
                const bf16x8 wf1 = unpack8(wv[j].y);
                const bf16x8 wf2 = unpack8(wv[j].z);
                const bf16x8 wf3 = unpack8(wv[j].w);
#pragma unroll
                for (int sb = 0; sb < NSUB; ++sb) {
                    if (sb * 16 >= nvalid)
                        break;                      // inactive subtile (wave-uniform)
                    u32x4 xa[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        xa[i] = u32x4{0u, 0u, 0u, 0u};
                        if (aval[sb])
                            xa[i] = *reinterpret_cast<const u32x4 *>(aptr[sb] + (size_t)g * kGroup + i * 8);
                    }
                    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
                    bf16x8 af;
                    af = permute_act(xa[0]);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, wf0, acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, neg136, acc, 0, 0, 0);
                    af = permute_act(xa[1]);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, wf1, acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, neg136, acc, 0, 0, 0);
                    af = permute_act(xa[2]);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, wf2, acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, neg136, acc, 0, 0, 0);
                    af = permute_act(xa[3]);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, wf3, acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, neg136, acc, 0, 0, 0);
                    tot[sb].x = __builtin_fmaf(sc[j], acc.x, tot[sb].x);
                    tot[sb].y = __builtin_fmaf(sc[j], acc.y, tot[sb].y);
                    tot[sb].z = __builtin_fmaf(sc[j], acc.z, tot[sb].z);
                    tot[sb].w = __builtin_fmaf(sc[j], acc.w, tot[sb].w);
                }
            }
        }

        // ---- cross-wave reduction through LDS ----
        // result lane layout: token (within subtile) = 4*kq + i, weight row = n16
#pragma unroll
        for (int sb = 0; sb < NSUB; ++sb) {
            s_red[wave][sb * 16 + kq * 4 + 0][n16] = tot[sb].x;
            s_red[wave][sb * 16 + kq * 4 + 1][n16] = tot[sb].y;
            s_red[wave][sb * 16 + kq * 4 + 2][n16] = tot[sb].z;
            s_red[wave][sb * 16 + kq * 4 + 3][n16] = tot[sb].w;
        }
        __syncthreads();
        if (KIND == MOE_GEMM_W13_SWIGLU) {
            for (int m = tid; m < nvalid; m += NWAVES * 64) {
                uint32_t packed[4];
#pragma unroll
                for (int jp = 0; jp < 4; ++jp) {
                    float hv[2];
#pragma unroll
                    for (int q = 0; q < 2; ++q) {
                        const int f = jp * 2 + q;
                        float gsum = 0.f, usum = 0.f;
#pragma unroll
                        for (int w = 0; w < NWAVES; ++w) {
                            gsum += s_red[w][m][f];
                            usum += s_red[w][m][8 + f];
                        }
                        hv[q] = silu(gsum) * usum;
                    }
                    packed[jp] = pack_bf16x2(hv[0], hv[1]);
                }
                uint16_t *dst = static_cast<uint16_t *>(p.c) + (size_t)(row0 + m) * p.ldc + tile * 8;
                *reinterpret_cast<u32x4 *>(dst) = u32x4{packed[0], packed[1], packed[2], packed[3]};
            }
        } else {
            for (int idx = tid; idx < nvalid * 2; idx += NWAVES * 64) {
                const int m = idx >> 1;
                const int h8 = (idx & 1) * 8;
                float v[8];
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    float sum = 0.f;
#pragma unroll
                    for (int w = 0; w < NWAVES; ++w)
                        sum += s_red[w][m][h8 + q];
                    v[q] = sum;
                }
                const size_t off = (size_t)(row0 + m) * p.ldc + tile * 16 + h8;
                if (p.c_f32) {
                    float *dst = static_cast<float *>(p.c) + off;
                    *reinterpret_cast<floatx4 *>(dst) = floatx4{v[0], v[1], v[2], v[3]};
                    *reinterpret_cast<floatx4 *>(dst + 4) = floatx4{v[4], v[5], v[6], v[7]};
                } else {
                    uint16_t *dst = static_cast<uint16_t *>(p.c) + off;
                    *reinterpret_cast<u32x4 *>(dst) =
                        u32x4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                              pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
                }
            }
        }
        __syncthreads();
    }
}

template <int KIND, int NWAVES, int NSUB>
hipError_t launch_cfg(const GemmArgs &a, int max_rows, hipStream_t st)
{
    constexpr int CS = 16 * NSUB;
    // upper bound on chunks: every non-empty expert adds at most one partial chunk
    const long long chunks = (long long)min(a.num_experts, max_rows) + max_rows / CS;
    const long long items = chunks * a.row_tiles;
    const long long cap = (long long)device_cu_count() * (NWAVES >= 8 ? 2 : 16 / NWAVES);
    long long grid = items < cap ? items : cap;
    if (grid < 1)
        grid = 1;
    hipLaunchKernelGGL((gemm_w4a16_kernel<KIND, NWAVES, NSUB, 4>), dim3((unsigned)grid),
                       dim3(NWAVES * 64), 0, st, a);
    return hipGetLastError();
}

template <int KIND>
hipError_t launch_kind(const GemmArgs &a, int max_rows, int nwaves, int nsub, hipStream_t st)
{
#define MOE_CFG(W, S)                                              \
    if (nwaves == W && nsub == S)                                  \
        return launch_cfg<KIND, W, S>(a, max_rows, st);
    MOE_CFG(1, 1) MOE_CFG(1, 2) MOE_CFG(1, 4)
    MOE_CFG(2, 1) MOE_CFG(2, 2) MOE_CFG(2, 4)
    MOE_CFG(4, 1) MOE_CFG(4, 2) MOE_CFG(4, 4)
    MOE_CFG(8, 1) MOE_CFG(8, 2) MOE_CFG(8, 4)
#undef MOE_CFG
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_grouped_gemm(const GemmLaunch &g, hipStream_t st)
{
    GemmArgs a;
    a.a = g.a;
    a.a_row_index = g.a_row_index;
    a.offsets = g.offsets;
    a.wq = g.wq;
    a.s = g.s;
    a.c = g.c;
    a.top_k = g.top_k;
    a.num_experts = g.num_experts;
    a.K = g.K;
    a.N = g.N;
    a.c_f32 = g.c_f32 ? 1 : 0;
    a.half = g.N / 2;
    if (g.kind == MOE_GEMM_W13_SWIGLU) {
        a.ldc = g.N / 2;
        a.row_tiles = g.N / 16;   // 8 features = 16 rows (8 gate + 8 up) per tile
    } else {
        a.ldc = g.N;
        a.row_tiles = g.N / 16;
    }
    const int G = g.K / kGroup;
    // K split: about four 128-groups per wave
    int nwaves = 1;
    while (nwaves < 8 && G / (nwaves * 2) >= 3)
        nwaves *= 2;
    // token subtiles per chunk from the mean rows per active expert
    const int mean_rows = g.expected_rows / (g.num_experts > 0 ? g.num_experts : 1);
    int nsub = mean_rows > 24 ? 4 : (mean_rows > 8 ? 2 : 1);
    if (const char *env = getenv("MOE_GEMM_NSUB"))
        nsub = atoi(env);
    if (const char *env = getenv("MOE_GEMM_NWAVES"))
        nwaves = atoi(env);
    if (g.kind == MOE_GEMM_W13_SWIGLU)
        return launch_kind<MOE_GEMM_W13_SWIGLU>(a, g.max_rows, nwaves, nsub, st);
    return launch_kind<MOE_GEMM_W2>(a, g.max_rows, nwaves, nsub, st);
}

}  // namespace moe

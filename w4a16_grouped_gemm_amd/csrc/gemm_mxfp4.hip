// gemm_mxfp4.hip -- the W4A4 variant: MXFP4 activations and weights on the
// gfx950 block-scaled matrix unit.
//
// Pages: FlashInfer PR #7196 analysis, section 2 ("Arithmetic Alignment":
// W4A4 finalizers beside the W4A16 ones) and its performance section (a
// W4A4 kernel beside the W4A16 one); GC-MoE abstract (FP4 block-scaled
// grouped GEMMs, 4-bit operands decoded in the matrix unit, activations
// requantized between the GEMMs). The pages fix no FP4 encoding; the format
// is the OCP MX one, MXFP4: E2M1 elements (magnitudes 0, 0.5, 1, 1.5, 2, 3,
// 4, 6) with one E8M0 scale 2^(s-127) per 32 elements along K.
//
// gfx950 design:
//  * v_mfma_scale_f32_16x16x128_f8f6f4 with both operands in FP4: lane l
//    holds 32 consecutive K elements (16 bytes, element k of the lane in
//    nibble k % 8 of dword k / 8) of row / column l % 16 of K block l / 16,
//    and one scale byte for them. That is the storage layout itself (two
//    elements per byte, even k in the low nibble, rows K-contiguous) and the
//    MX block of 32, so codes and scales go from memory to the matrix unit
//    unchanged: one MFMA per 16x16 tile and 128 K, no unpack, no scale FMA.
//  * Operand A = 16 routed rows of one expert (the activations), operand B =
//    16 weight rows; the result lane holds 4 rows x 1 weight row, as in the
//    W4A16 kernels, so the SwiGLU and row-index epilogue is the same.
//  * Code loads use the default cache policy: a lane's 16 bytes are a
//    quarter of a row's 64 bytes of one group, so each 128-byte line holds two
//    groups of a row, and the streaming (non-temporal) policy let lines go
//    before their second half was read (measured on MI355X, Qwen3-30B-A3B
//    gate/up at 256 tokens: 305 MB fetched for 210 MB of data, 58.5 us;
//    default policy 228 MB, 54.7 us).
//  * K <= 2048 (mx_gemm_lds_kernel): each item stages its chunk's
//    activation codes and scales for the whole K in LDS once (coalesced row
//    reads), the four waves read their fragments there, the weight scales of
//    a tile are loaded once per item, and only the weight codes stream
//    through a register ring. Per-wave gathers of 16 activation rows and of
//    16 rows' scale bytes for every group had made the address unit the
//    bottleneck (Qwen3-30B-A3B gate/up at 256 tokens: 82 -> 55 us).
//  * Larger K (mx_gemm_kernel): everything streams HBM -> VGPR (codes 16
//    bytes per lane and group, the group's four scale bytes as one dword),
//    no LDS staging and no barrier in the K loop.
//  * Work items (expert chunk of up to 16 NSUB rows, block of 4 waves x TPW
//    tiles) come from the chunk prefix over `offsets`, as in the W4A16
//    streaming kernel.
//  * mx_quantize_kernel: one thread per 32-element block: the block maximum,
//    the shared exponent floor(log2 amax) - 2 (clamped to the E8M0 range),
//    and each element / 2^e rounded to the nearest E2M1 value with ties to
//    the even code and saturation at 6, by comparisons against the midpoints
//    (exact in binary32: the division by a power of two is exact).
#include "gemm_core.hpp"
#include "mx_quant.hpp"
#include "route_core.hpp"

#include <map>
#include <mutex>
#include <utility>

namespace moe {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));

struct MxArgs {
    const uint8_t *a;            // activation codes [rows][K/2]
    const uint8_t *as;           // activation scales [rows][K/32]
    const int32_t *a_row_index;  // row r reads a row a_row_index[r] / top_k (NULL: row r)
    uint32_t a_bytes, as_bytes;
    const int32_t *offsets;      // [E+1]
    const uint8_t *wq;           // weight codes [E][N][K/2]
    const uint8_t *ws;           // weight scales [E][N][K/32]
    void *c;
    const int32_t *c_row_index;  // output row of result row r (NULL: r)
    uint32_t c_row_bytes;
    int top_k, num_experts, K, N, ldc, half, c_f32;
    int w_tiled;                 // codes tiled: tile t, group g at ((t/8)*G*8 + t%8)*1 KiB + g*8 KiB
    uint8_t *cq, *cs;            // non-NULL (SwiGLU, LDS kernel): h stored as MXFP4 codes and scales
    // non-NULL (LDS kernel): the permutation is built in LDS from these
    // routing ids (offsets and a_row_index unused); workgroup 0 stores its tables
    const int32_t *ids;
    int T, begin;
    int32_t *cnt_out, *off_out, *perm_out, *inv_out;
    // the W4A4 layer's small-batch path (LDS kernel, SRC != MX_SRC_CHUNKS):
    // items from a slot table, built by routing inside the gate/up GEMM
    // (which also quantizes the tokens' x rows while staging them) or read
    // from the stored table (down); rows are slots t*k + j
    const float *logits;         // [T][E_g]
    int E_g;
    const uint16_t *x;           // bf16 x [T][K] (gate/up)
    int32_t *slot_ids;           // [T*k]: global expert id of each slot (gate/up writes, down reads)
    float *slot_w;               // [T*k]: routing weight (gate/up writes)
    int32_t *pres;               // [T*k]: the slot if its expert is local, else -1
};

// Item sources of the LDS kernel: the chunk prefix (offsets or the routing
// ids), the small-batch slot table built by routing in the kernel, or the
// stored slot table.
enum { MX_SRC_CHUNKS = 0, MX_SRC_ROUTE = 1, MX_SRC_SLOTS = 2 };

// Lane offset of tile `tile`'s codes (row `row` of the plain layout) and the
// byte step from one 128-wide group to the next.
__device__ __forceinline__ uint32_t mx_code_offset(const MxArgs &p, int tile, uint32_t row, int lane, int kq)
{
    if (p.w_tiled)
        return (uint32_t)((tile >> 3) * (p.K >> 7) * 8 + (tile & 7)) * 1024u + (uint32_t)lane * 16u;
    return row * (uint32_t)(p.K >> 1) + (uint32_t)kq * 16u;
}
__device__ __forceinline__ uint32_t mx_group_stride(const MxArgs &p) { return p.w_tiled ? 8192u : 64u; }

__device__ __forceinline__ floatx4 mfma_fp4(u32x4 a, uint32_t sa, u32x4 b, uint32_t sb, floatx4 c)
{
    const v8i va = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
    const v8i vb = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(va, vb, c, 4, 4, 0, (int)sa, 0, (int)sb);
}

template <int KIND>
__device__ __forceinline__ uint32_t mx_tile_row(const MxArgs &p, int tile, int n16)
{
    if (KIND == MOE_GEMM_W13_SWIGLU)
        return (uint32_t)(n16 < 8 ? tile * 8 + n16 : p.half + tile * 8 + (n16 - 8));
    return (uint32_t)(tile * 16 + n16);
}

// Epilogue of one item: result lane (n16, kq) holds rows 4kq + i of weight
// row n16 of each (tile, subtile); SwiGLU pairs gate row n16 with up row
// n16 + 8 (lane n16 ^ 8).
template <int KIND, int TPW, int NSUB>
__device__ __forceinline__ void mx_store(const MxArgs &p, const floatx4 (&acc)[TPW][NSUB], int tile0, int row0,
                                         int nvalid, int nsub, int n16, int kq, const int *s_orow = nullptr)
{
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(p.c_row_index, p.c_row_bytes);
#pragma unroll
    for (int sb = 0; sb < NSUB; ++sb) {
        if (sb >= nsub)
            break;
        int orow[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = sb * 16 + kq * 4 + i;
            const int r = row0 + min(m, nvalid - 1);
            orow[i] = s_orow ? s_orow[min(m, nvalid - 1)]
                    : p.c_row_index ? (int)__builtin_amdgcn_raw_buffer_load_b32(rc, (uint32_t)r * 4u, 0, 0) : r;
        }
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            const floatx4 v = acc[t][sb];
            const float rr[4] = {v.x, v.y, v.z, v.w};
            if (KIND == MOE_GEMM_W13_SWIGLU) {
                float u[4];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    u[i] = row_swap8(rr[i]);
                if (n16 < 8) {
                    uint16_t *c = static_cast<uint16_t *>(p.c);
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (sb * 16 + kq * 4 + i < nvalid)
                            c[(size_t)orow[i] * p.ldc + (tile0 + t) * 8 + n16] =
                                (uint16_t)f32_to_bf16_rne(silu_fast(rr[i]) * u[i]);
                }
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (sb * 16 + kq * 4 + i < nvalid) {
                        const size_t off = (size_t)orow[i] * p.ldc + (tile0 + t) * 16 + n16;
                        if (p.c_f32)
                            static_cast<float *>(p.c)[off] = rr[i];
                        else
                            static_cast<uint16_t *>(p.c)[off] = (uint16_t)f32_to_bf16_rne(rr[i]);
                    }
                }
            }
        }
    }
}

// Epilogue of one item with bf16 output, through LDS: each wave writes two
// tiles of a subtile (16 rows x 16 columns each) to its own 1 KiB of LDS,
// then every lane stores one 16-byte run of an output row (two lanes per
// tile row) instead of four scattered 2-byte values per tile. `s_area`: 4 KiB
// that no wave reads any more (the caller has passed a barrier).
constexpr int kMxStoreLdsBytes = 4 * 1024;

template <int TPW, int NSUB>
__device__ __forceinline__ void mx_store_lds(const MxArgs &p, const floatx4 (&acc)[TPW][NSUB], int tile0, int row0,
                                             int nvalid, int nsub, int n16, int kq, int wave, int lane,
                                             uint16_t *s_area, const int *s_orow)
{
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(p.c_row_index, p.c_row_bytes);
    uint16_t *so = s_area + wave * 512;
    uint16_t *c = static_cast<uint16_t *>(p.c);
    // lane: tile pair + lane / 32, row (lane / 2) % 16, columns 8 (lane % 2) ..
    const int rr = (lane >> 1) & 15, part = lane & 1, half = lane >> 5;
#pragma unroll
    for (int sb = 0; sb < NSUB; ++sb) {
        if (sb >= nsub)
            break;
        const int m = sb * 16 + rr;
        int orow = 0;
        if (m < nvalid)
            orow = s_orow ? s_orow[m]
                 : p.c_row_index ? (int)__builtin_amdgcn_raw_buffer_load_b32(rc, (uint32_t)(row0 + m) * 4u, 0, 0)
                                 : row0 + m;
#pragma unroll
        for (int t0 = 0; t0 < TPW; t0 += 2) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                if (t0 + u < TPW) {
                    const floatx4 v = acc[t0 + u][sb];
                    const float r4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        so[(u * 16 + kq * 4 + i) * 16 + n16] = (uint16_t)f32_to_bf16_rne(r4[i]);
                }
            }
            __builtin_amdgcn_wave_barrier();
            const int t = t0 + half;
            if (t < TPW && m < nvalid) {
                const u32x4 d = *reinterpret_cast<const u32x4 *>(so + (half * 16 + rr) * 16 + part * 8);
                *reinterpret_cast<u32x4 *>(c + (size_t)orow * p.ldc + (tile0 + t) * 16 + part * 8) = d;
            }
            __builtin_amdgcn_wave_barrier();             // the area is rewritten for the next pair
        }
    }
}

template <int TPW, int NSUB>
__host__ __device__ constexpr int mx_h_stride() { return 32 * TPW + 8; }   // bf16 elements per LDS row

// SwiGLU epilogue that stores h already requantized (the down GEMM's MXFP4
// activations): the item's bf16 h values, rounded as mx_store rounds them, go
// to an LDS tile of CS rows x 32 TPW features (s_h, over the staged
// activations), then each thread quantizes one row's block of 32 features
// with the shared block quantizer and stores its 16 code bytes and scale
// byte: the same bits as storing bf16 h and quantizing it afterwards.
template <int TPW, int NSUB>
__device__ __forceinline__ void mx_store_quant(const MxArgs &p, const floatx4 (&acc)[TPW][NSUB], int block, int row0,
                                               int nvalid, int nsub, int n16, int kq, int wave, int tid,
                                               uint16_t *s_h, const int *s_orow = nullptr)
{
    constexpr int CS = 16 * NSUB, HST = mx_h_stride<TPW, NSUB>();
    __syncthreads();                                   // every wave is done with the staged activations
#pragma unroll
    for (int sb = 0; sb < NSUB; ++sb) {
        if (sb >= nsub)
            break;
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            const floatx4 v = acc[t][sb];
            const float rr[4] = {v.x, v.y, v.z, v.w};
            float u[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                u[i] = row_swap8(rr[i]);               // partner lane holds the up row
            if (n16 < 8) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    s_h[(sb * 16 + kq * 4 + i) * HST + (wave * TPW + t) * 8 + n16] =
                        (uint16_t)f32_to_bf16_rne(silu_fast(rr[i]) * u[i]);
            }
        }
    }
    __syncthreads();
    const int ldq = p.ldc >> 1, lds_ = p.ldc >> 5;     // bytes per h row: codes, scales
    for (int q = tid; q < CS * TPW; q += 256) {
        const int r = q / TPW, b = q - r * TPW;
        if (r < nvalid) {
            const uint32_t *src = reinterpret_cast<const uint32_t *>(s_h + r * HST + b * 32);
            uint32_t w[16];
#pragma unroll
            for (int d = 0; d < 16; ++d)
                w[d] = src[d];
            uint32_t out[4];
            const uint32_t sc = mx_quant_block(w, out);
            const int orow = s_orow ? s_orow[r] : p.c_row_index ? p.c_row_index[row0 + r] : row0 + r;
            const int f0 = block * 32 * TPW + b * 32;  // first feature of the block
            *reinterpret_cast<u32x4 *>(p.cq + (size_t)orow * ldq + (f0 >> 1)) = u32x4{out[0], out[1], out[2], out[3]};
            p.cs[(size_t)orow * lds_ + (f0 >> 5)] = (uint8_t)sc;
        }
    }
}

template <int KIND, int TPW, int NSUB, int RING>
__global__ __launch_bounds__(256) void mx_gemm_kernel(MxArgs p)
{
    constexpr int CS = 16 * NSUB;
    constexpr int BT = 4 * TPW;
    extern __shared__ __align__(16) unsigned char s_dyn[];
    const int E = p.num_experts;
    int *s_prefix = reinterpret_cast<int *>(s_dyn);
    int *s_wtot = s_prefix + (E + 1);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, n16 = lane & 15, kq = lane >> 4;
    build_chunk_prefix<256>(p.offsets, 0, E, CS, s_prefix, s_wtot);

    const int ntiles = p.N >> 4;
    const int nblocks = ntiles / BT;
    const int total_items = s_prefix[E] * nblocks;
    const int G = p.K / kGroup;
    const uint32_t row_bytes = (uint32_t)(p.K >> 1), srow_bytes = (uint32_t)(p.K >> 5);
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.a, p.a_bytes);
    const __amdgpu_buffer_rsrc_t ras = make_rsrc(p.as, p.as_bytes);
    const uint32_t sh = 8u * (uint32_t)kq;             // this lane's scale byte within a group's dword
    const int nx = (int)gridDim.x >= kXcds ? kXcds : 1;  // XCD-aware item ranges, as in the W4A16 kernels
    const int xcd = blockIdx.x % nx;
    const int i_end = (int)((long long)total_items * (xcd + 1) / nx);
    for (int item = (int)((long long)total_items * xcd / nx) + blockIdx.x / nx; item < i_end;
         item += gridDim.x / nx) {
        const int chunk = item / nblocks;
        const int block = item - chunk * nblocks;
        const int e = uniform(chunk_expert(s_prefix, E, chunk));
        const int row0 = uniform(p.offsets[e] + (chunk - s_prefix[e]) * CS);
        const int nvalid = uniform(min(CS, p.offsets[e + 1] - row0));
        const int nsub = (nvalid + 15) >> 4;
        const int tile0 = block * BT + wave * TPW;
        const uint32_t wbytes = (uint32_t)p.N * row_bytes, wsbytes = (uint32_t)p.N * srow_bytes;
        const __amdgpu_buffer_rsrc_t rw = make_rsrc(p.wq + (size_t)e * wbytes, wbytes);
        const __amdgpu_buffer_rsrc_t rws = make_rsrc(p.ws + (size_t)e * wsbytes, wsbytes);
        uint32_t vw[TPW], vws[TPW];
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            const uint32_t row = mx_tile_row<KIND>(p, tile0 + t, n16);
            vw[t] = mx_code_offset(p, tile0 + t, row, lane, kq);
            vws[t] = row * srow_bytes;
        }
        const uint32_t gstride = mx_group_stride(p);
        uint32_t va[NSUB], vas[NSUB];
#pragma unroll
        for (int sb = 0; sb < NSUB; ++sb) {
            const int m = sb * 16 + n16;
            const int r = row0 + min(m, nvalid - 1);
            const uint32_t src = p.a_row_index ? (uint32_t)(p.a_row_index[r] / p.top_k) : (uint32_t)r;
            const bool ok = m < nvalid;
            va[sb] = ok ? src * row_bytes + (uint32_t)kq * 16u : kOutOfRange;
            vas[sb] = ok ? src * srow_bytes : kOutOfRange;
        }
        floatx4 acc[TPW][NSUB];
#pragma unroll
        for (int t = 0; t < TPW; ++t)
#pragma unroll
            for (int sb = 0; sb < NSUB; ++sb)
                acc[t][sb] = floatx4{0.f, 0.f, 0.f, 0.f};
        u32x4 wv[RING][TPW], av[RING][NSUB];
        uint32_t wsv[RING][TPW], asv[RING][NSUB];
        // group g -> ring slot g % RING; groups past G read out of range (zeros)
        auto load = [&](int g, int b) {
            const uint32_t oor = g < G ? 0u : kOutOfRange;
            const uint32_t gc = (uint32_t)(g < G ? g : 0);
#pragma unroll
            for (int t = 0; t < TPW; ++t) {
                wv[b][t] = bload16_codes<false>(rw, vw[t] | oor, gc * gstride);
                wsv[b][t] = __builtin_amdgcn_raw_buffer_load_b32(rws, vws[t] | oor, gc * 4u, 0);
            }
#pragma unroll
            for (int sb = 0; sb < NSUB; ++sb) {
                av[b][sb] = bload16(ra, va[sb] | oor, gc * 64u);
                asv[b][sb] = __builtin_amdgcn_raw_buffer_load_b32(ras, vas[sb] | oor, gc * 4u, 0);
            }
        };
#pragma unroll
        for (int r = 0; r < RING - 1; ++r)
            load(r, r);
        for (int g0 = 0; g0 < G; g0 += RING) {
#pragma unroll
            for (int j = 0; j < RING; ++j) {
                const int g = g0 + j;
                load(g + RING - 1, (j + RING - 1) % RING);
                if (g < G) {
#pragma unroll
                    for (int sb = 0; sb < NSUB; ++sb) {
                        if (sb < nsub) {
#pragma unroll
                            for (int t = 0; t < TPW; ++t)
                                acc[t][sb] = mfma_fp4(av[j][sb], asv[j][sb] >> sh, wv[j][t], wsv[j][t] >> sh,
                                                      acc[t][sb]);
                        }
                    }
                }
            }
        }
        mx_store<KIND, TPW, NSUB>(p, acc, tile0, row0, nvalid, nsub, n16, kq);
    }
}

// The same items with the chunk's activations staged in LDS: the 16*NSUB
// rows' codes and scales for the whole K are copied once per item, rows
// contiguous (coalesced global reads, one row segment per 64 lanes), and the
// four waves read their MFMA fragments from there, instead of each wave
// gathering 16 rows per load instruction for every group. The weight scales
// of a tile's 16 rows are loaded once per item (lane (n16, kq): the dwords of
// groups 4kq .. 4kq+3 of row n16) and each group's byte is taken from the
// owning lane with ds_bpermute. Only weight codes stream through the
// register ring. K <= 2048 (16 groups: one 16-byte scale load per lane).
// Row strides: K/2 + 16 bytes for codes (a 16-row fragment read spreads over
// all banks), K/32 + 4 for scales.
__host__ __device__ constexpr int mx_code_stride(int K) { return K / 2 + 16; }
__host__ __device__ constexpr int mx_scale_stride(int K) { return K / 32 + 4; }
constexpr int kMxStageBatch = 8;                     // staging loads a thread issues before storing
constexpr int kMxQuantBatch = 4;                     // x blocks a thread loads before quantizing (small batch)

template <int KIND, int TPW, int NSUB, int RING, int SRC = MX_SRC_CHUNKS, int PL = 8>
__global__ __launch_bounds__(256) void mx_gemm_lds_kernel(MxArgs p)
{
    static_assert(SRC == MX_SRC_CHUNKS || NSUB == 1, "small-batch items hold at most 16 rows");
    constexpr int CS = 16 * NSUB;
    constexpr int BT = 4 * TPW;
    extern __shared__ __align__(16) unsigned char s_dyn[];
    const int E = p.num_experts;
    const int K = p.K, G = K / kGroup;
    const int AST = mx_code_stride(K), ASS = mx_scale_stride(K);
    uint8_t *s_a = s_dyn;                                        // [CS][AST]
    uint8_t *s_as = s_a + CS * AST;                              // [CS][ASS]
    // the staging area also holds the requantizing epilogue's h tile
    const int stage = max(CS * (AST + ASS), CS * mx_h_stride<TPW, NSUB>() * 2);
    int *s_src = reinterpret_cast<int *>(s_dyn + stage);         // [CS] activation row of each chunk row
    int *s_orow = s_src + CS;                                    // [CS] small batch: output row (slot)
    int *s_prefix = s_orow + CS;                                 // [E+1] chunk prefix
    int *s_off = s_prefix + (E + 1);                             // [E+1] expert row offsets
    int *s_wtot = s_off + (E + 1);                               // [8] scan scratch
    uint16_t *s_row = reinterpret_cast<uint16_t *>(s_wtot + 8);  // ids: slot of each permuted row
    // small-batch slot tables, in the same region
    int *s_loc = s_prefix;                                       // [kDecMaxSlots] local expert per slot, -1
    int *s_lead = s_loc + kDecMaxSlots;                          // [kDecMaxSlots] leaders in slot order
    int *s_nlead = s_lead + kDecMaxSlots;                        // [4]
    int *s_first = s_nlead + 4;                                  // [E] each expert's first slot
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, n16 = lane & 15, kq = lane >> 4;
    const int S_slots = p.T * p.top_k;
    const int ntiles = p.N >> 4;
    const int nblocks = ntiles / BT;
    int total_items;
    if constexpr (SRC == MX_SRC_CHUNKS) {
        if (p.ids) {
            // the permutation from the routing ids; its scratch is the staging area
            uint32_t *s_bits = reinterpret_cast<uint32_t *>(s_dyn);
            int *s_wpre = reinterpret_cast<int *>(s_bits + E * ((p.T + 31) >> 5));
            const IdsTables it{p.ids, p.T, p.top_k, p.begin, E, p.cnt_out, p.off_out, p.perm_out, p.inv_out};
            build_from_ids<256>(it, CS, s_bits, s_wpre, s_row, s_prefix, s_off, s_wtot);
        } else {
            build_chunk_prefix<256>(p.offsets, 0, E, CS, s_prefix, s_wtot, s_off);
        }
        total_items = s_prefix[E] * nblocks;
    } else {
        // the small-batch slot table, as the W4A16 streaming kernel builds it
        for (int e = tid; e < E; e += 256)
            s_first[e] = kDecMaxSlots;
        if constexpr (SRC == MX_SRC_ROUTE) {
            // every workgroup routes all tokens: one DPP row of 16 lanes per
            // token, or a whole wave per token while there are at most four
            // (the k rounds of the selection are the routing's serial part; 64
            // lanes hold a quarter of the logits each; the same selection and
            // weights bit for bit, the weights formed in lanes 0..k-1)
            auto keep = [&](int t, int q, int eg, float wt) {
                if (q < p.top_k) {
                    const int sl = t * p.top_k + q;
                    const int le = eg - p.begin;
                    const int loc = (le >= 0 && le < E) ? le : -1;
                    s_loc[sl] = loc;
                    if (blockIdx.x == 0) {
                        p.slot_ids[sl] = eg;
                        p.slot_w[sl] = wt;
                        p.pres[sl] = loc >= 0 ? sl : -1;
                    }
                }
            };
            if (p.T <= 4) {
                if (wave < p.T) {
                    int eg;
                    float wt;
                    route_token<64, (PL >= 4 ? PL / 4 : 1)>(p.logits + (size_t)wave * p.E_g, p.E_g, p.top_k, lane, eg,
                                                           wt);
                    keep(wave, lane, eg, wt);
                }
            } else {
                for (int t0 = wave * 4; t0 < p.T; t0 += 16) {
                    const int t = t0 + (lane >> 4);
                    if (t < p.T) {
                        int eg;
                        float wt;
                        route_token<16, PL>(p.logits + (size_t)t * p.E_g, p.E_g, p.top_k, n16, eg, wt);
                        keep(t, n16, eg, wt);
                    }
                }
            }
        } else {
            for (int sl = tid; sl < S_slots; sl += 256)
                s_loc[sl] = p.pres[sl] >= 0 ? p.slot_ids[sl] - p.begin : -1;
        }
        __syncthreads();
        build_leaders<256>(S_slots, E, s_loc, s_first, s_lead, s_nlead);
        total_items = s_nlead[0] * nblocks;
    }
    const uint32_t row_bytes = (uint32_t)(K >> 1), srow_bytes = (uint32_t)(K >> 5);
    const int ppr = K >> 5;                                      // 16-byte code pieces per row
    const int spr = K >> 7;                                      // scale dwords per row
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.a, p.a_bytes);
    const __amdgpu_buffer_rsrc_t ras = make_rsrc(p.as, p.as_bytes);
    const uint32_t sh = 8u * (uint32_t)kq;
    const int nx = (int)gridDim.x >= kXcds ? kXcds : 1;
    const int xcd = blockIdx.x % nx;
    const int i_end = (int)((long long)total_items * (xcd + 1) / nx);
    for (int item = (int)((long long)total_items * xcd / nx) + blockIdx.x / nx; item < i_end;
         item += gridDim.x / nx) {
        const int chunk = item / nblocks;
        const int block = item - chunk * nblocks;
        int e, row0, nvalid;
        uint64_t m0 = 0, m1 = 0;                                 // small batch: the expert's slots
        if constexpr (SRC == MX_SRC_CHUNKS) {
            e = uniform(chunk_expert(s_prefix, E, chunk));
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
        const uint32_t wbytes = (uint32_t)p.N * row_bytes, wsbytes = (uint32_t)p.N * srow_bytes;
        const __amdgpu_buffer_rsrc_t rw = make_rsrc(p.wq + (size_t)e * wbytes, wbytes);
        const __amdgpu_buffer_rsrc_t rws = make_rsrc(p.ws + (size_t)e * wsbytes, wsbytes);
        // activation row of chunk row tid (gather index read now, stored after
        // the barrier); small batch: row m is the m-th slot, its output row
        int src = 0, orow = 0;
        if (tid < CS && tid < nvalid) {
            if constexpr (SRC == MX_SRC_CHUNKS) {
                src = p.ids ? s_row[row0 + tid] / p.top_k
                            : p.a_row_index ? p.a_row_index[row0 + tid] / p.top_k : row0 + tid;
            } else {
                orow = nth_slot(m0, m1, tid);
                src = SRC == MX_SRC_ROUTE ? orow / p.top_k : orow;   // gate/up: the slot's token
            }
        }
        // weight scales of this wave's tiles, and the first RING-1 groups of codes
        uint32_t vw[TPW];
        u32x4 wsc[TPW];
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            const uint32_t row = mx_tile_row<KIND>(p, tile0 + t, n16);
            vw[t] = mx_code_offset(p, tile0 + t, row, lane, kq);
            // dword d of the lane: group 4kq + d (dwords past G are not read:
            // a row's scales end inside the lane's 16 bytes when G % 4 != 0)
            const uint32_t so = row * srow_bytes + (uint32_t)kq * 16u;
            uint32_t d4[4];
#pragma unroll
            for (int d = 0; d < 4; ++d)
                d4[d] = __builtin_amdgcn_raw_buffer_load_b32(rws, 4 * kq + d < G ? so + 4u * d : kOutOfRange, 0, 0);
            wsc[t] = u32x4{d4[0], d4[1], d4[2], d4[3]};
        }
        u32x4 wv[RING][TPW];
        const uint32_t gstride = mx_group_stride(p);
        auto load_w = [&](int g, int b) {
            const uint32_t oor = g < G ? 0u : kOutOfRange;
            const uint32_t gc = (uint32_t)(g < G ? g : 0);
#pragma unroll
            for (int t = 0; t < TPW; ++t)
                wv[b][t] = bload16_codes<false>(rw, vw[t] | oor, gc * gstride);
        };
#pragma unroll
        for (int r = 0; r < RING - 1; ++r)
            load_w(r, r);
        __syncthreads();                                         // the previous item is done with s_a
        if (tid < CS) {
            s_src[tid] = src;
            s_orow[tid] = orow;
        }
        __syncthreads();
        if constexpr (SRC == MX_SRC_ROUTE) {
            // the rows' bf16 x, quantized here (the quantize kernel's bits)
            // into the staging layout: block b of row r -> codes s_a[r][16b..],
            // scale s_as[r][b]; every load of a batch before any store
            const int nb = K >> 5;
            for (int base = 0; base < nvalid * nb; base += kMxQuantBatch * 256) {
                uint32_t w[kMxQuantBatch][16];
#pragma unroll
                for (int u = 0; u < kMxQuantBatch; ++u) {
                    const int q = base + u * 256 + tid;
                    if (q < nvalid * nb) {
                        const int r = q / nb, b = q - r * nb;
                        const u32x4 *xs4 = reinterpret_cast<const u32x4 *>(p.x + (size_t)s_src[r] * K + b * 32);
#pragma unroll
                        for (int c = 0; c < 4; ++c) {
                            const u32x4 d = xs4[c];
                            w[u][4 * c] = d.x;
                            w[u][4 * c + 1] = d.y;
                            w[u][4 * c + 2] = d.z;
                            w[u][4 * c + 3] = d.w;
                        }
                    }
                }
#pragma unroll
                for (int u = 0; u < kMxQuantBatch; ++u) {
                    const int q = base + u * 256 + tid;
                    if (q < nvalid * nb) {
                        const int r = q / nb, b = q - r * nb;
                        uint32_t out[4];
                        s_as[r * ASS + b] = (uint8_t)mx_quant_block(w[u], out);
                        *reinterpret_cast<u32x4 *>(s_a + r * AST + b * 16) = u32x4{out[0], out[1], out[2], out[3]};
                    }
                }
            }
        }
        // stage the chunk's codes and scales: a batch of loads per thread goes
        // out before any is stored (rows past nvalid are left as they are:
        // their results are never stored)
        for (int base = 0; base < (SRC == MX_SRC_ROUTE ? 0 : nvalid * ppr); base += kMxStageBatch * 256) {
            u32x4 v[kMxStageBatch];
            uint32_t sv[kMxStageBatch / 4];
#pragma unroll
            for (int u = 0; u < kMxStageBatch; ++u) {
                const int q = base + u * 256 + tid;
                const int r = q / ppr, c = q - r * ppr;
                const uint32_t off = q < nvalid * ppr ? (uint32_t)s_src[min(r, CS - 1)] * row_bytes + (uint32_t)c * 16u
                                                      : kOutOfRange;
                v[u] = bload16(ra, off, 0);
            }
            // scale dwords: one per 4 code pieces (spr = ppr / 4)
#pragma unroll
            for (int u = 0; u < kMxStageBatch / 4; ++u) {
                const int q = base / 4 + u * 256 + tid;
                const int r = q / spr, c = q - r * spr;
                const bool ok = q < min(nvalid * spr, (base + kMxStageBatch * 256) / 4);
                sv[u] = __builtin_amdgcn_raw_buffer_load_b32(
                    ras, ok ? (uint32_t)s_src[min(r, CS - 1)] * srow_bytes + (uint32_t)c * 4u : kOutOfRange, 0, 0);
            }
#pragma unroll
            for (int u = 0; u < kMxStageBatch; ++u) {
                const int q = base + u * 256 + tid;
                const int r = q / ppr, c = q - r * ppr;
                if (q < nvalid * ppr)
                    *reinterpret_cast<u32x4 *>(s_a + r * AST + c * 16) = v[u];
            }
#pragma unroll
            for (int u = 0; u < kMxStageBatch / 4; ++u) {
                const int q = base / 4 + u * 256 + tid;
                const int r = q / spr, c = q - r * spr;
                if (q < min(nvalid * spr, (base + kMxStageBatch * 256) / 4))
                    *reinterpret_cast<uint32_t *>(s_as + r * ASS + c * 4) = sv[u];
            }
        }
        __syncthreads();

        floatx4 acc[TPW][NSUB];
#pragma unroll
        for (int t = 0; t < TPW; ++t)
#pragma unroll
            for (int sb = 0; sb < NSUB; ++sb)
                acc[t][sb] = floatx4{0.f, 0.f, 0.f, 0.f};
        for (int g0 = 0; g0 < G; g0 += RING) {
#pragma unroll
            for (int j = 0; j < RING; ++j) {
                const int g = g0 + j;
                load_w(g + RING - 1, (j + RING - 1) % RING);
                if (g < G) {
                    // weight scale byte kq of (row n16, group g): lane n16 + 16 (g / 4), dword g % 4
                    const int src_lane = (n16 + 16 * (g >> 2)) * 4;
                    uint32_t wsg[TPW];
#pragma unroll
                    for (int t = 0; t < TPW; ++t) {
                        const int gq = g & 3;
                        const uint32_t d = gq == 0 ? wsc[t].x : gq == 1 ? wsc[t].y : gq == 2 ? wsc[t].z : wsc[t].w;
                        wsg[t] = (uint32_t)__builtin_amdgcn_ds_bpermute(src_lane, (int)d) >> sh;
                    }
#pragma unroll
                    for (int sb = 0; sb < NSUB; ++sb) {
                        if (sb < nsub) {
                            const int m = sb * 16 + n16;
                            const u32x4 a = *reinterpret_cast<const u32x4 *>(s_a + m * AST + g * 64 + kq * 16);
                            const uint32_t as = *reinterpret_cast<const uint32_t *>(s_as + m * ASS + g * 4) >> sh;
#pragma unroll
                            for (int t = 0; t < TPW; ++t)
                                acc[t][sb] = mfma_fp4(a, as, wv[j][t], wsg[t], acc[t][sb]);
                        }
                    }
                }
            }
        }
        const int *orows = SRC == MX_SRC_CHUNKS ? nullptr : s_orow;
        if (KIND == MOE_GEMM_W13_SWIGLU && p.cq)
            mx_store_quant<TPW, NSUB>(p, acc, block, row0, nvalid, nsub, n16, kq, wave, tid,
                                      reinterpret_cast<uint16_t *>(s_a), orows);
        else if (KIND != MOE_GEMM_W13_SWIGLU && !p.c_f32 && kMxStoreLdsBytes <= stage) {
            __syncthreads();                                     // every wave is done with the staged rows
            mx_store_lds<TPW, NSUB>(p, acc, tile0, row0, nvalid, nsub, n16, kq, wave, lane,
                                    reinterpret_cast<uint16_t *>(s_a), orows);
        } else
            mx_store<KIND, TPW, NSUB>(p, acc, tile0, row0, nvalid, nsub, n16, kq, orows);
    }
}

// rows x (K/32) blocks; `rows_dev` (nullable) bounds the rows on the device.
__global__ __launch_bounds__(256) void mx_quantize_kernel(long long rows, int K, const uint16_t *__restrict__ x,
                                                          uint8_t *__restrict__ codes, uint8_t *__restrict__ scales,
                                                          const int32_t *__restrict__ rows_dev)
{
    const int nb = K >> 5;
    const long long R = rows_dev ? (long long)rows_dev[0] : rows;
    const long long total = (R < rows ? R : rows) * nb;
    for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (long long)gridDim.x * blockDim.x) {
        const u32x4 *src = reinterpret_cast<const u32x4 *>(x + i * 32);
        uint32_t w[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const u32x4 d = src[q];
            w[4 * q] = d.x;
            w[4 * q + 1] = d.y;
            w[4 * q + 2] = d.z;
            w[4 * q + 3] = d.w;
        }
        uint32_t out[4];
        scales[i] = (uint8_t)mx_quant_block(w, out);
        *reinterpret_cast<u32x4 *>(codes + i * 16) = u32x4{out[0], out[1], out[2], out[3]};
    }
}

template <typename F>
int mx_resident_per_cu(F kernel, size_t lds)
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

template <int KIND, int TPW, int NSUB, int RING>
hipError_t mx_launch(const MxArgs &a, int max_rows, hipStream_t st)
{
    auto kernel = mx_gemm_kernel<KIND, TPW, NSUB, RING>;
    const size_t lds = sizeof(int) * (a.num_experts + 1 + 4);
    const int per_cu = mx_resident_per_cu(kernel, lds);
    const int nblocks = (a.N >> 4) / (4 * TPW);
    const long long chunks = (long long)min(a.num_experts, max_rows) + max_rows / (16 * NSUB);
    long long grid = chunks * nblocks;
    const long long cap = (long long)device_cu_count() * per_cu;
    grid = grid < cap ? grid : cap;
    grid = grid < 1 ? 1 : grid;
    if (grid >= kXcds)
        grid -= grid % kXcds;
    hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(256), lds, st, a);
    return hipGetLastError();
}

// The LDS-staged kernel when the whole K of a chunk fits (K <= 2048, the
// one-load weight scales), else the register-streaming one.
// LDS of the LDS-staged kernel: the staging area (also the requantizing
// epilogue's tile and the permutation scratch), then the tables; `slots`:
// T * k with the permutation built from the ids, else 0.
template <int TPW, int NSUB>
size_t mx_stage_bytes(int K)
{
    constexpr int CS = 16 * NSUB;
    const size_t a = (size_t)CS * (mx_code_stride(K) + mx_scale_stride(K));
    const size_t h = (size_t)CS * mx_h_stride<TPW, NSUB>() * 2;    // the requantizing epilogue's tile
    return a > h ? a : h;
}

template <int TPW, int NSUB>
size_t mx_lds_bytes(int K, int num_experts, int slots)
{
    constexpr int CS = 16 * NSUB;
    const size_t chunk_tables = sizeof(int) * (2 * (num_experts + 1) + 8) + 2 * (size_t)slots;
    const size_t slot_tables = sizeof(int) * (2 * kDecMaxSlots + 4 + num_experts);   // small batch
    return mx_stage_bytes<TPW, NSUB>(K) + sizeof(int) * 2 * CS +
           (chunk_tables > slot_tables ? chunk_tables : slot_tables);
}

// Whether the LDS-staged kernel takes the launch (K <= 2048, the one-load
// weight scales, and its LDS); with the permutation built from the ids, also
// whether its scratch fits the staging area.
template <int TPW, int NSUB>
bool mx_lds_fits(int K, int num_experts, int T = 0, int slots = 0)
{
    if (K > 2048 || mx_lds_bytes<TPW, NSUB>(K, num_experts, slots) > 150 * 1024)
        return false;
    return slots == 0 || (num_experts <= 256 && slots <= kIdsPerThread * 256 &&
                          ids_scratch_bytes(num_experts, T) <= mx_stage_bytes<TPW, NSUB>(K));
}

template <int KIND, int TPW, int NSUB, int RING>
hipError_t mx_launch_any(const MxArgs &a, int max_rows, hipStream_t st)
{
    constexpr int CS = 16 * NSUB;
    const int slots = a.ids ? a.T * a.top_k : 0;
    const size_t lds = mx_lds_bytes<TPW, NSUB>(a.K, a.num_experts, slots);
    if (!mx_lds_fits<TPW, NSUB>(a.K, a.num_experts, a.T, slots)) {
        if (a.ids)
            return hipErrorInvalidValue;                 // mx_gemm_ids_supported() rules this out
        return mx_launch<KIND, TPW, NSUB, RING>(a, max_rows, st);
    }
    auto kernel = mx_gemm_lds_kernel<KIND, TPW, NSUB, RING>;
    static std::once_flag once;
    std::call_once(once, [&] {
        (void)hipFuncSetAttribute(reinterpret_cast<const void *>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                                  150 * 1024);
    });
    const int per_cu = mx_resident_per_cu(kernel, lds);
    const int nblocks = (a.N >> 4) / (4 * TPW);
    const long long chunks = (long long)min(a.num_experts, max_rows) + max_rows / CS;
    long long grid = chunks * nblocks;
    const long long cap = (long long)device_cu_count() * per_cu;
    grid = grid < cap ? grid : cap;
    grid = grid < 1 ? 1 : grid;
    if (grid >= kXcds)
        grid -= grid % kXcds;
    hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(256), lds, st, a);
    return hipGetLastError();
}

// The LDS kernel with a small-batch item source (at most one item per
// expert and weight block).
template <int KIND, int TPW, int SRC, int PL>
hipError_t mx_launch_small(const MxArgs &a, int max_rows, hipStream_t st)
{
    auto kernel = mx_gemm_lds_kernel<KIND, TPW, 1, 4, SRC, PL>;
    const size_t lds = mx_lds_bytes<TPW, 1>(a.K, a.num_experts, 0);
    static std::once_flag once;
    std::call_once(once, [&] {
        (void)hipFuncSetAttribute(reinterpret_cast<const void *>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                                  150 * 1024);
    });
    const int per_cu = mx_resident_per_cu(kernel, lds);
    const int nblocks = (a.N >> 4) / (4 * TPW);
    long long grid = (long long)min(a.num_experts, max_rows) * nblocks;
    const long long cap = (long long)device_cu_count() * per_cu;
    grid = grid < cap ? grid : cap;
    grid = grid < 1 ? 1 : grid;
    if (grid >= kXcds)
        grid -= grid % kXcds;
    hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(256), lds, st, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_mx_quantize(long long rows, int K, const uint16_t *x, uint8_t *codes, uint8_t *scales,
                              const int32_t *rows_dev, hipStream_t st)
{
    const long long blocks_total = rows * (K / 32);
    long long grid = (blocks_total + 255) / 256;
    const long long cap = (long long)device_cu_count() * 8;
    grid = grid < cap ? grid : cap;
    grid = grid < 1 ? 1 : grid;
    hipLaunchKernelGGL(mx_quantize_kernel, dim3((unsigned)grid), dim3(256), 0, st, rows, K, x, codes, scales, rows_dev);
    return hipGetLastError();
}

// Tiling of an MXFP4 grouped GEMM: rows per active expert under uniform
// routing pick one subtile for decode, four (64-row chunks) once experts hold
// many rows; tiles per wave from how many items the grid gets.
static void mx_choose(const MxGemmLaunch &g, int &tpw, int &nsub)
{
    const double E = g.num_experts > 0 ? g.num_experts : 1;
    const double R = g.expected_rows > 0 ? g.expected_rows : 1;
    const double T = g.max_rows / (double)(g.top_k > 0 ? g.top_k : 1);
    const double ps = R / (T * E);
    const double active = E * (1.0 - pow(1.0 - (ps < 1.0 ? ps : 1.0), T));
    const double m = R / (active > 1.0 ? active : 1.0);
    const int ntiles = g.N / 16;
    nsub = m > 40.0 ? 4 : m > 12.0 ? 2 : 1;
    tpw = 4;
    const double chunks = fmax(active, R / (16.0 * nsub));
    while (tpw > 1 && (ntiles % (4 * tpw) != 0 || chunks * ntiles / tpw <= 2.0 * device_cu_count()))
        tpw >>= 1;
}

static MxArgs mx_args(const MxGemmLaunch &g);

// The W4A4 layer's small-batch path: the tiling mx_choose picks with one
// subtile (at most 16 rows per expert), on the LDS kernel.
static bool mx_small_tiling(const MxGemmLaunch &g, int &tpw)
{
    int nsub;
    mx_choose(g, tpw, nsub);
    if (g.c_f32 || (g.N / 16) % (4 * tpw) != 0)
        return false;
    if (tpw == 4)
        return mx_lds_fits<4, 1>(g.K, g.num_experts);
    if (tpw == 2)
        return mx_lds_fits<2, 1>(g.K, g.num_experts);
    return mx_lds_fits<1, 1>(g.K, g.num_experts);
}

bool mx_small_supported(const MxGemmLaunch &g)
{
    int tpw;
    return mx_small_tiling(g, tpw);
}

hipError_t launch_mx_small(const MxGemmLaunch &g, const MxSmallSource &src, hipStream_t st)
{
    int tpw;
    if (!mx_small_tiling(g, tpw) || src.T * g.top_k > kDecMaxSlots || src.E_g > 256 ||
        (g.kind == MOE_GEMM_W13_SWIGLU) != (src.logits != nullptr))
        return hipErrorInvalidValue;
    MxArgs a = mx_args(g);
    a.T = src.T;
    a.begin = src.begin;
    a.logits = src.logits;
    a.E_g = src.E_g;
    a.x = src.x;
    a.slot_ids = src.ids;
    a.slot_w = src.w;
    a.pres = src.pres;
    a.a_row_index = nullptr;
    a.c_row_index = nullptr;
    const int R = g.max_rows;
    if (g.kind == MOE_GEMM_W13_SWIGLU) {
#define MOE_MXS_ROUTE(TP)                                                                                    \
        if (tpw == TP)                                                                                      \
            return src.E_g <= 64    ? mx_launch_small<MOE_GEMM_W13_SWIGLU, TP, MX_SRC_ROUTE, 4>(a, R, st)   \
                   : src.E_g <= 128 ? mx_launch_small<MOE_GEMM_W13_SWIGLU, TP, MX_SRC_ROUTE, 8>(a, R, st)   \
                                    : mx_launch_small<MOE_GEMM_W13_SWIGLU, TP, MX_SRC_ROUTE, 16>(a, R, st);
        MOE_MXS_ROUTE(1) MOE_MXS_ROUTE(2) MOE_MXS_ROUTE(4)
#undef MOE_MXS_ROUTE
    } else if (g.kind == MOE_GEMM_W2) {
        if (tpw == 1)
            return mx_launch_small<MOE_GEMM_W2, 1, MX_SRC_SLOTS, 8>(a, R, st);
        if (tpw == 2)
            return mx_launch_small<MOE_GEMM_W2, 2, MX_SRC_SLOTS, 8>(a, R, st);
        if (tpw == 4)
            return mx_launch_small<MOE_GEMM_W2, 4, MX_SRC_SLOTS, 8>(a, R, st);
    }
    return hipErrorInvalidValue;
}

bool mx_gemm_ids_supported(const MxGemmLaunch &g, int T)
{
    int tpw, nsub;
    mx_choose(g, tpw, nsub);
    const int slots = T * g.top_k;
    if (g.c_f32 || slots > g.max_rows || (g.N / 16) % (4 * tpw) != 0)
        return false;
#define MOE_MX_FITS(TP, NS) \
    if (tpw == TP && nsub == NS) return mx_lds_fits<TP, NS>(g.K, g.num_experts, T, slots);
    MOE_MX_FITS(1, 1) MOE_MX_FITS(2, 1) MOE_MX_FITS(4, 1) MOE_MX_FITS(1, 2) MOE_MX_FITS(2, 2) MOE_MX_FITS(4, 2)
    MOE_MX_FITS(1, 4) MOE_MX_FITS(2, 4) MOE_MX_FITS(4, 4)
#undef MOE_MX_FITS
    return false;
}

static MxArgs mx_args(const MxGemmLaunch &g)
{
    MxArgs a{};
    a.a = g.a;
    a.as = g.as;
    a.a_row_index = g.a_row_index;
    a.a_bytes = (uint32_t)((size_t)g.a_rows * (g.K / 2));
    a.as_bytes = (uint32_t)((size_t)g.a_rows * (g.K / 32));
    a.offsets = g.offsets;
    a.wq = g.wq;
    a.ws = g.ws;
    a.c = g.c;
    a.c_row_index = g.c_row_index;
    a.c_row_bytes = g.c_row_index ? (uint32_t)g.max_rows * 4u : 0u;
    a.top_k = g.top_k;
    a.num_experts = g.num_experts;
    a.K = g.K;
    a.N = g.N;
    a.half = g.N / 2;
    a.ldc = g.kind == MOE_GEMM_W13_SWIGLU ? g.N / 2 : g.N;
    a.c_f32 = g.c_f32 ? 1 : 0;
    a.w_tiled = g.w_tiled ? 1 : 0;
    a.cq = g.kind == MOE_GEMM_W13_SWIGLU ? g.cq : nullptr;
    a.cs = g.kind == MOE_GEMM_W13_SWIGLU ? g.cs : nullptr;
    return a;
}

hipError_t launch_mx_grouped_gemm(const MxGemmLaunch &g, hipStream_t st)
{
    MxArgs a = mx_args(g);
    if (g.ids) {
        if (!mx_gemm_ids_supported(g, g.T))
            return hipErrorInvalidValue;
        a.ids = g.ids;
        a.T = g.T;
        a.begin = g.begin;
        a.cnt_out = g.counts_out;
        a.off_out = g.offsets_out;
        a.perm_out = g.perm_out;
        a.inv_out = g.inv_perm_out;
        a.a_row_index = nullptr;
    }
    int tpw, nsub;
    mx_choose(g, tpw, nsub);
    if ((g.N / 16) % (4 * tpw) != 0)
        return hipErrorInvalidValue;                   // N is a multiple of 128: 4 waves x 2 tiles always divide
    auto go = [&](auto kindc) -> hipError_t {
        constexpr int KIND = decltype(kindc)::value;
        // h requantized in the epilogue where the LDS kernel runs; otherwise
        // bf16 h, then the quantize kernel over the routed rows (same bits)
#define MOE_MX(TP, NS)                                                                                      \
        if (tpw == TP && nsub == NS) {                                                                      \
            if (a.cq && !mx_lds_fits<TP, NS>(a.K, a.num_experts, a.T, a.ids ? a.T * a.top_k : 0)) {        \
                MxArgs b = a;                                                                               \
                b.cq = nullptr;                                                                             \
                b.cs = nullptr;                                                                             \
                const hipError_t e = mx_launch_any<KIND, TP, NS, (NS == 4 ? 2 : 4)>(b, g.max_rows, st);    \
                if (e != hipSuccess)                                                                        \
                    return e;                                                                               \
                return launch_mx_quantize(g.max_rows, a.ldc, static_cast<const uint16_t *>(a.c), a.cq, a.cs, \
                                          g.offsets + g.num_experts, st);                                   \
            }                                                                                               \
            return mx_launch_any<KIND, TP, NS, (NS == 4 ? 2 : 4)>(a, g.max_rows, st);                       \
        }
        MOE_MX(1, 1) MOE_MX(2, 1) MOE_MX(4, 1) MOE_MX(1, 2) MOE_MX(2, 2) MOE_MX(4, 2) MOE_MX(1, 4) MOE_MX(2, 4)
        MOE_MX(4, 4)
#undef MOE_MX
        return hipErrorInvalidValue;
    };
    if (g.kind == MOE_GEMM_W13_SWIGLU)
        return go(std::integral_constant<int, MOE_GEMM_W13_SWIGLU>());
    if (g.kind == MOE_GEMM_W2)
        return go(std::integral_constant<int, MOE_GEMM_W2>());
    return go(std::integral_constant<int, MOE_GEMM_W13_RAW>());
}

}  // namespace moe

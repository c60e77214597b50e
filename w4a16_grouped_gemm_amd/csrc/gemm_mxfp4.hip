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
};

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
                                         int nvalid, int nsub, int n16, int kq)
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
            orow[i] = p.c_row_index ? (int)__builtin_amdgcn_raw_buffer_load_b32(rc, (uint32_t)r * 4u, 0, 0) : r;
        }
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            const floatx4 v = acc[t][sb];
            const float rr[4] = {v.x, v.y, v.z, v.w};
            if (KIND == MOE_GEMM_W13_SWIGLU) {
                float u[4];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    u[i] = __shfl_xor(rr[i], 8, 64);
                if (n16 < 8) {
                    uint16_t *c = static_cast<uint16_t *>(p.c);
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (sb * 16 + kq * 4 + i < nvalid)
                            c[(size_t)orow[i] * p.ldc + (tile0 + t) * 8 + n16] =
                                (uint16_t)f32_to_bf16_rne(silu(rr[i]) * u[i]);
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

// SwiGLU epilogue that stores h already requantized (the down GEMM's MXFP4
// activations): the item's bf16 h values, rounded as mx_store rounds them, go
// to an LDS tile of CS rows x 32 TPW features (s_h, over the staged
// activations), then each thread quantizes one row's block of 32 features
// with the shared block quantizer and stores its 16 code bytes and scale
// byte: the same bits as storing bf16 h and quantizing it afterwards.
template <int TPW, int NSUB>
__host__ __device__ constexpr int mx_h_stride() { return 32 * TPW + 8; }   // bf16 elements per LDS row

template <int TPW, int NSUB>
__device__ __forceinline__ void mx_store_quant(const MxArgs &p, const floatx4 (&acc)[TPW][NSUB], int block, int row0,
                                               int nvalid, int nsub, int n16, int kq, int wave, int tid,
                                               uint16_t *s_h)
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
                u[i] = __shfl_xor(rr[i], 8, 64);       // partner lane holds the up row
            if (n16 < 8) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    s_h[(sb * 16 + kq * 4 + i) * HST + (wave * TPW + t) * 8 + n16] =
                        (uint16_t)f32_to_bf16_rne(silu(rr[i]) * u[i]);
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
            const int orow = p.c_row_index ? p.c_row_index[row0 + r] : row0 + r;
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

template <int KIND, int TPW, int NSUB, int RING>
__global__ __launch_bounds__(256) void mx_gemm_lds_kernel(MxArgs p)
{
    constexpr int CS = 16 * NSUB;
    constexpr int BT = 4 * TPW;
    extern __shared__ __align__(16) unsigned char s_dyn[];
    const int E = p.num_experts;
    const int K = p.K, G = K / kGroup;
    const int AST = mx_code_stride(K), ASS = mx_scale_stride(K);
    uint8_t *s_a = s_dyn;                                        // [CS][AST]
    uint8_t *s_as = s_a + CS * AST;                              // [CS][ASS]
    int *s_src = reinterpret_cast<int *>(s_as + CS * ASS);       // [CS] activation row of each chunk row
    int *s_prefix = s_src + CS;                                  // [E+1] chunk prefix
    int *s_off = s_prefix + (E + 1);                             // [E+1] expert row offsets
    int *s_wtot = s_off + (E + 1);                               // [8] scan scratch
    uint16_t *s_row = reinterpret_cast<uint16_t *>(s_wtot + 8);  // ids: slot of each permuted row
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, n16 = lane & 15, kq = lane >> 4;
    if (p.ids) {
        // the permutation from the routing ids; its scratch is the staging area
        uint32_t *s_bits = reinterpret_cast<uint32_t *>(s_dyn);
        int *s_wpre = reinterpret_cast<int *>(s_bits + E * ((p.T + 31) >> 5));
        const IdsTables it{p.ids, p.T, p.top_k, p.begin, E, p.cnt_out, p.off_out, p.perm_out, p.inv_out};
        build_from_ids<256>(it, CS, s_bits, s_wpre, s_row, s_prefix, s_off, s_wtot);
    } else {
        build_chunk_prefix<256>(p.offsets, 0, E, CS, s_prefix, s_wtot, s_off);
    }

    const int ntiles = p.N >> 4;
    const int nblocks = ntiles / BT;
    const int total_items = s_prefix[E] * nblocks;
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
        const int e = uniform(chunk_expert(s_prefix, E, chunk));
        const int row0 = uniform(s_off[e] + (chunk - s_prefix[e]) * CS);
        const int nvalid = uniform(min(CS, s_off[e + 1] - row0));
        const int nsub = (nvalid + 15) >> 4;
        const int tile0 = block * BT + wave * TPW;
        const uint32_t wbytes = (uint32_t)p.N * row_bytes, wsbytes = (uint32_t)p.N * srow_bytes;
        const __amdgpu_buffer_rsrc_t rw = make_rsrc(p.wq + (size_t)e * wbytes, wbytes);
        const __amdgpu_buffer_rsrc_t rws = make_rsrc(p.ws + (size_t)e * wsbytes, wsbytes);
        // activation row of chunk row tid (gather index read now, stored after the barrier)
        int src = 0;
        if (tid < CS && tid < nvalid)
            src = p.ids ? s_row[row0 + tid] / p.top_k
                        : p.a_row_index ? p.a_row_index[row0 + tid] / p.top_k : row0 + tid;
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
        if (tid < CS)
            s_src[tid] = src;
        __syncthreads();
        // stage the chunk's codes and scales: a batch of loads per thread goes
        // out before any is stored (rows past nvalid are left as they are:
        // their results are never stored)
        for (int base = 0; base < nvalid * ppr; base += kMxStageBatch * 256) {
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
        if (KIND == MOE_GEMM_W13_SWIGLU && p.cq)
            mx_store_quant<TPW, NSUB>(p, acc, block, row0, nvalid, nsub, n16, kq, wave, tid,
                                      reinterpret_cast<uint16_t *>(s_a));
        else
            mx_store<KIND, TPW, NSUB>(p, acc, tile0, row0, nvalid, nsub, n16, kq);
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
size_t mx_lds_bytes(int K, int num_experts, int slots)
{
    constexpr int CS = 16 * NSUB;
    size_t stage = (size_t)CS * (mx_code_stride(K) + mx_scale_stride(K) + 4);
    const size_t h = (size_t)CS * mx_h_stride<TPW, NSUB>() * 2;    // the requantizing epilogue's tile
    stage = stage > h ? stage : h;
    return stage + sizeof(int) * (2 * (num_experts + 1) + 8) + 2 * (size_t)slots;
}

// Whether the LDS-staged kernel takes the launch (K <= 2048, the one-load
// weight scales, and its LDS); with the permutation built from the ids, also
// whether its scratch fits the staging area.
template <int TPW, int NSUB>
bool mx_lds_fits(int K, int num_experts, int T = 0, int slots = 0)
{
    constexpr int CS = 16 * NSUB;
    if (K > 2048 || mx_lds_bytes<TPW, NSUB>(K, num_experts, slots) > 150 * 1024)
        return false;
    return slots == 0 || (num_experts <= 256 && slots <= kIdsPerThread * 256 &&
                          ids_scratch_bytes(num_experts, T) <= (size_t)CS * (mx_code_stride(K) + mx_scale_stride(K)));
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

hipError_t launch_mx_grouped_gemm(const MxGemmLaunch &g, hipStream_t st)
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

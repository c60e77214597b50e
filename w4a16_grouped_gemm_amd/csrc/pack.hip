// pack.hip -- plain -> tiled reordering of int4 weight codes.
//
// The grouped GEMM's wave loads 16 bytes per lane: lane l holds 32 codes
// (one 128-wide group's quarter) of weight row l%16 of a 16-row tile. In the
// plain row-major layout those 64 lanes touch 16 rows x 64 bytes; the tiled
// layout stores exactly those 1 KiB contiguously, and the 8 tiles of a block
// next to each other for each group, so a workgroup streams its weights as
// one sequential run. Inside each word the codes are reordered so that they
// unpack in column order (activations are then used as they lie in memory). FlashInfer PR #7196 analysis, section 3, likewise keeps
// a kernel-internal weight layout that its tests invert back to a plain one.
#include "common.hpp"

namespace moe {

namespace {

// Nibbles of one little-endian word: even codes (columns 0,2,4,6) to nibbles
// 0..3, odd codes (1,3,5,7) to nibbles 4..7. The GEMM's unpack pairs nibble j
// with nibble j + 4, which are then the adjacent columns 2j and 2j + 1.
__device__ __forceinline__ uint32_t shuffle_word(uint32_t d)
{
    auto squeeze = [](uint32_t x) {                   // low nibble of each byte -> 16 bits
        x = (x | (x >> 4)) & 0x00FF00FFu;
        return (x | (x >> 8)) & 0x0000FFFFu;
    };
    return squeeze(d & 0x0F0F0F0Fu) | (squeeze((d >> 4) & 0x0F0F0F0Fu) << 16);
}

// One thread per 16-byte unit of the output: unit u of expert e is
// (((b * G + g) * 8 + i) * 64 + l), read from plain row row(16*(8b+i), l%16),
// bytes [64g + 16(l/16), +16), each word shuffled (int4 codes) or as it is
// (MXFP4 codes: a lane's 16 bytes already are its matrix-unit operand).
__global__ __launch_bounds__(256) void pack_kernel(int E, int N, int K, int half, int pair_rows, int shuffle,
                                                   const uint8_t *__restrict__ src, uint8_t *__restrict__ dst)
{
    const int G = K / kGroup;
    const long long row_bytes = K / 2;
    const long long per_expert = (long long)N * row_bytes / 16;
    const long long total = per_expert * E;
    for (long long u = (long long)blockIdx.x * blockDim.x + threadIdx.x; u < total;
         u += (long long)gridDim.x * blockDim.x) {
        const int e = (int)(u / per_expert);
        long long r = u - (long long)e * per_expert;
        const int l = (int)(r & 63);
        r >>= 6;
        const int i = (int)(r & 7);
        r >>= 3;
        const int g = (int)(r % G);
        const int b = (int)(r / G);
        const int tile = 8 * b + i;
        const int n = l & 15;
        const int row = pair_rows ? (n < 8 ? 8 * tile + n : half + 8 * tile + n - 8) : 16 * tile + n;
        const uint8_t *s = src + ((long long)e * N + row) * row_bytes + 64 * g + 16 * (l >> 4);
        const u32x4 v = *reinterpret_cast<const u32x4 *>(s);
        *reinterpret_cast<u32x4 *>(dst + u * 16) =
            shuffle ? u32x4{shuffle_word(v.x), shuffle_word(v.y), shuffle_word(v.z), shuffle_word(v.w)} : v;
    }
}

}  // namespace

hipError_t launch_pack_weights(int E, int N, int K, int half, bool pair_rows, const uint8_t *wq,
                               uint8_t *wq_tiled, hipStream_t st, bool shuffle)
{
    const long long total = (long long)E * N * (K / 2) / 16;
    long long blocks = (total + 255) / 256;
    const long long cap = (long long)device_cu_count() * 16;
    if (blocks > cap)
        blocks = cap;
    if (blocks < 1)
        blocks = 1;
    hipLaunchKernelGGL(pack_kernel, dim3((unsigned)blocks), dim3(256), 0, st, E, N, K, half, pair_rows ? 1 : 0,
                       shuffle ? 1 : 0, wq, wq_tiled);
    return hipGetLastError();
}

}  // namespace moe

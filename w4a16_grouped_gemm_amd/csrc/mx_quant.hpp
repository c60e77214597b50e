// mx_quant.hpp -- the MXFP4 block quantizer shared by every kernel that
// quantizes activations (the standalone quantize kernel, the gate/up GEMM's
// requantizing epilogue, the routing launch that also quantizes x), so that
// all of them produce the same codes and scales bit for bit.
//
// Format (the OCP MX reading of the pages' W4A4 variant: FlashInfer PR #7196
// analysis, section 2, W4A4 finalizers; GC-MoE abstract, activations
// requantized between the GEMMs): 32 consecutive elements share one E8M0
// scale 2^(s-127); each element is an E2M1 code (sign, 2 exponent bits, 1
// mantissa bit: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6).
#pragma once

#include "common.hpp"

namespace moe {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// One block of 32 bf16 values (w[q] holds elements 2q and 2q + 1, low half
// first) -> 16 bytes of codes (element k in nibble k % 8 of dword k / 8) and
// the E8M0 scale byte: the shared exponent floor(log2 amax) - 2 (clamped to
// the E8M0 range; an all-zero block takes 2^-127), each element / 2^e rounded
// to the nearest E2M1 value (0, 0.5, 1, 1.5, 2, 3, 4, 6; a midpoint to the
// even code, past 6 to 6, a NaN or infinity to 6 with its sign).
// The rounding is gfx950's scaled FP4 conversion (two bf16 elements -> one
// code byte, divided by the scale operand): on every bf16 value, at scales
// 2^-127 .. 2^127 (2^-127 a binary32 subnormal), it gives exactly the codes
// of the midpoint comparisons above, NaN and infinity included (measured on
// MI355X against that rule). The division by a power of two is exact, and a
// finite block's elements / 2^e stay below 8.
__device__ __forceinline__ uint32_t mx_quant_block(const uint32_t (&w)[16], uint32_t (&out)[4])
{
    // the block maximum on the magnitude bits (bf16 orders like its magnitude)
    uint32_t amax = 0;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        const uint32_t lo = w[q] & 0x7FFFu, hi = (w[q] >> 16) & 0x7FFFu;
        amax = lo > amax ? lo : amax;
        amax = hi > amax ? hi : amax;
    }
    int ex = -127;
    if (amax != 0) {
        const int bexp = (int)(amax >> 7);              // biased exponent of the bf16 maximum
        const int fl = bexp > 0 ? bexp - 127 : -133 + (31 - __builtin_clz(amax & 0x7Fu));   // floor(log2)
        ex = fl - 2;
        ex = ex < -127 ? -127 : (ex > 127 ? 127 : ex);
    }
    // 2^ex as a binary32 value: normal from 2^-126 on, 2^-127 the subnormal
    // 0x00400000 (a finite bf16 maximum gives ex <= 125)
    const float scale = __uint_as_float(ex >= -126 ? (uint32_t)(ex + 127) << 23 : 0x00400000u);
#pragma unroll
    for (int d = 0; d < 4; ++d)
        out[d] = 0u;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        // elements 2q, 2q + 1 -> byte q % 4 of dword q / 4 (low nibble first);
        // with a zero destination and byte 0 selected the result's other bits are 0
        const uint32_t byte = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(0u, __builtin_bit_cast(bf16x2, w[q]), scale, 0);
        out[q >> 2] |= byte << (8 * (q & 3));
    }
    return (uint32_t)(ex + 127);
}

// Quantizing a row-major bf16 array of nblk 32-element blocks (rows of K
// elements, K a multiple of 32: block i is elements 32i .. 32i + 31, its codes
// bytes 16i .. 16i + 15, its scale byte i) inside another kernel: a thread
// loads its blocks i0, i0 + stride, ... (NB of them) first, does other work
// while they are in flight, then quantizes and stores them.
template <int NB>
__device__ __forceinline__ void mx_blocks_load(const uint16_t *x, long long nblk, long long i0, long long stride,
                                               uint32_t (&w)[NB][16])
{
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        const long long i = i0 + j * stride;
        if (i < nblk) {
            const u32x4 *src = reinterpret_cast<const u32x4 *>(x + i * 32);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const u32x4 d = src[q];
                w[j][4 * q] = d.x;
                w[j][4 * q + 1] = d.y;
                w[j][4 * q + 2] = d.z;
                w[j][4 * q + 3] = d.w;
            }
        }
    }
}

template <int NB>
__device__ __forceinline__ void mx_blocks_store(const uint32_t (&w)[NB][16], long long nblk, long long i0,
                                                long long stride, uint8_t *codes, uint8_t *scales)
{
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        const long long i = i0 + j * stride;
        if (i < nblk) {
            uint32_t out[4];
            scales[i] = (uint8_t)mx_quant_block(w[j], out);
            *reinterpret_cast<u32x4 *>(codes + i * 16) = u32x4{out[0], out[1], out[2], out[3]};
        }
    }
}

// Every block from i0 on in steps of stride: the first NB from w (already
// loaded), the rest in batches of NB.
template <int NB>
__device__ __forceinline__ void mx_blocks_finish(uint32_t (&w)[NB][16], const uint16_t *x, long long nblk,
                                                 long long i0, long long stride, uint8_t *codes, uint8_t *scales)
{
    mx_blocks_store<NB>(w, nblk, i0, stride, codes, scales);
    for (long long b = i0 + NB * stride; b < nblk; b += NB * stride) {
        mx_blocks_load<NB>(x, nblk, b, stride, w);
        mx_blocks_store<NB>(w, nblk, b, stride, codes, scales);
    }
}

}  // namespace moe

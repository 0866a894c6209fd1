// w4a16_device.h — device-side helpers shared by the W4A16 HIP kernels
// (gfx950 / CDNA4, wave64).  Private to this library.
//
// Packed format ([QUANT] sub-section 3 listing, widened to 32-bit words): word
// j of a row holds elements 8j..8j+7, element 8j+i in bits 4i..4i+3 as the
// offset-binary code q+8.  Sources are cited by the keys of include/w4a16.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a16 {

constexpr int kGroup = 128;         // elements per scale, along K
constexpr int kWave = 64;           // CDNA wavefront width
constexpr int kChunkElems = 32;     // one 16-byte packed load = 4 words = 32 codes
constexpr int kChunksPerGroup = kGroup / kChunkElems;

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ half2_t as_h2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }
__device__ __forceinline__ uint32_t as_u32(half2_t h) { return __builtin_bit_cast(uint32_t, h); }

__device__ __forceinline__ float f16_bits_to_f32(uint16_t b) {
    return (float)__builtin_bit_cast(_Float16, b);
}
// fp32 -> fp16 bits, round to nearest even (the default rounding mode).
__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
    return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// Activation pairing used by every kernel.  A packed word's codes are
// unpacked two at a time as (n0,n4), (n1,n5), (n2,n6), (n3,n7) — nibble i
// and nibble i+4 sit in the two 16-bit halves of the word — so activations
// are staged in the same order: for an 8-element block x0..x7 the four
// half2 values (x0,x4), (x1,x5), (x2,x6), (x3,x7).  `lo` holds (x0,x1),(x2,x3)
// and `hi` holds (x4,x5),(x6,x7) as loaded.
__device__ __forceinline__ uint4 pair_block(uint32_t x01, uint32_t x23, uint32_t x45,
                                            uint32_t x67) {
    uint4 p;
    p.x = __builtin_amdgcn_perm(x45, x01, 0x05040100u);  // (x0, x4)
    p.y = __builtin_amdgcn_perm(x45, x01, 0x07060302u);  // (x1, x5)
    p.z = __builtin_amdgcn_perm(x67, x23, 0x05040100u);  // (x2, x6)
    p.w = __builtin_amdgcn_perm(x67, x23, 0x07060302u);  // (x3, x7)
    return p;
}

// Sum of the activations a chunk pairs with low-nibble (bits 0-3 of each
// byte) and high-nibble codes, from a chunk of 4 paired blocks.
// Returns (sum over x0,x4,x2,x6 ; sum over x1,x5,x3,x7) of the 4 blocks.
__device__ __forceinline__ float2 chunk_sums(const uint4 (&p)[4]) {
    const half2_t one = {(_Float16)1.0f, (_Float16)1.0f};
    float lo = 0.f, hi = 0.f;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        lo = __builtin_amdgcn_fdot2(as_h2(p[b].x), one, lo, false);
        lo = __builtin_amdgcn_fdot2(as_h2(p[b].z), one, lo, false);
        hi = __builtin_amdgcn_fdot2(as_h2(p[b].y), one, hi, false);
        hi = __builtin_amdgcn_fdot2(as_h2(p[b].w), one, hi, false);
    }
    return make_float2(lo, hi);
}

// Dot product of one packed word (8 codes) with its paired activations,
// codes taken as raw nibbles n = q + 8 read as fp16 subnormals:
//   (w & 0x000F000F) is the half2 (n0, n4) * 2^-24,
//   (w & 0x00F000F0) is the half2 (n1, n5) * 2^-20,
// and the same for (w >> 8).  Two accumulators keep the two scalings:
//   lo += 2^-24 * sum n x over nibbles 0,4,2,6;  hi += 2^-20 * sum over 1,5,3,7.
// The offset 8 is removed once per chunk from the activation sums.
__device__ __forceinline__ void dot_word_nibbles(uint32_t w, const uint4& xp, float& lo,
                                                 float& hi) {
    const uint32_t w8 = w >> 8;
    lo = __builtin_amdgcn_fdot2(as_h2(w & 0x000F000Fu), as_h2(xp.x), lo, false);
    hi = __builtin_amdgcn_fdot2(as_h2(w & 0x00F000F0u), as_h2(xp.y), hi, false);
    lo = __builtin_amdgcn_fdot2(as_h2(w8 & 0x000F000Fu), as_h2(xp.z), lo, false);
    hi = __builtin_amdgcn_fdot2(as_h2(w8 & 0x00F000F0u), as_h2(xp.w), hi, false);
}

// One packed word -> its 8 dequantized weights fp16(s*q) as 4 half2 in the
// paired order (w0,w4),(w1,w5),(w2,w6),(w3,w7).  0x6400|n is the fp16 value
// 1024+n, so (1024+n) - 1032 = n - 8 = q exactly; for the nibbles at bits
// 4-7 the value is 1024+16n and (1024+16n)/16 - 72 = q exactly.  The final
// product with the scale is rounded once (to nearest even).
__device__ __forceinline__ void dequant_word(uint32_t w, half2_t s2, half2_t (&out)[4]) {
    const half2_t m1032 = {(_Float16)-1032.0f, (_Float16)-1032.0f};
    const half2_t inv16 = {(_Float16)0.0625f, (_Float16)0.0625f};
    const half2_t m72 = {(_Float16)-72.0f, (_Float16)-72.0f};
    const uint32_t w8 = w >> 8;
    half2_t q0 = as_h2((w & 0x000F000Fu) | 0x64006400u) + m1032;
    half2_t q1 = __builtin_elementwise_fma(as_h2((w & 0x00F000F0u) | 0x64006400u), inv16, m72);
    half2_t q2 = as_h2((w8 & 0x000F000Fu) | 0x64006400u) + m1032;
    half2_t q3 = __builtin_elementwise_fma(as_h2((w8 & 0x00F000F0u) | 0x64006400u), inv16, m72);
    out[0] = q0 * s2;
    out[1] = q1 * s2;
    out[2] = q2 * s2;
    out[3] = q3 * s2;
}

}  // namespace w4a16

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

// Keeps a constant in a VGPR, opaque to the optimizer, so that
// (w & mask) | magic is selected as one v_and_or_b32 (gfx9 VOP3 encodings
// take no 32-bit literal, and two SGPR operands exceed the constant bus).
__device__ __forceinline__ uint32_t in_vgpr(uint32_t v) {
    asm volatile("" : "+v"(v));
    return v;
}

struct CodeConsts {
    uint32_t m_lo, m_hi, magic;
};
__device__ __forceinline__ CodeConsts code_consts() {
    return CodeConsts{in_vgpr(0x000F000Fu), in_vgpr(0x00F000F0u), in_vgpr(0x64006400u)};
}

// One packed word -> its 8 codes q = n - 8 as exact fp16 integers, in the
// paired order (q0,q4),(q1,q5),(q2,q6),(q3,q7).  0x6400|n is the fp16 value
// 1024+n, so (1024+n) - 1032 = q exactly; for the nibbles at bits 4-7 the
// value is 1024+16n and (1024+16n)/16 - 72 = q exactly.  Costs one shift,
// four v_and_or_b32 and four packed-fp16 add/fma.
__device__ __forceinline__ void codes_word(uint32_t w, const CodeConsts& k, half2_t (&q)[4]) {
    const half2_t m1032 = {(_Float16)-1032.0f, (_Float16)-1032.0f};
    const half2_t inv16 = {(_Float16)0.0625f, (_Float16)0.0625f};
    const half2_t m72 = {(_Float16)-72.0f, (_Float16)-72.0f};
    const uint32_t w8 = w >> 8;
    q[0] = as_h2((w & k.m_lo) | k.magic) + m1032;
    q[1] = __builtin_elementwise_fma(as_h2((w & k.m_hi) | k.magic), inv16, m72);
    q[2] = as_h2((w8 & k.m_lo) | k.magic) + m1032;
    q[3] = __builtin_elementwise_fma(as_h2((w8 & k.m_hi) | k.magic), inv16, m72);
}

// Asymmetric codes: n - zc for the nibbles n of one word, exact fp16
// integers in the paired order, with the bias constants -1024 - zc (low
// nibbles, after the 0x6400 trick) and -64 - zc (high nibbles, after the
// division by 16).  |zc| <= kZeroClamp keeps every operand and result an
// integer below 2^11.
constexpr int kZeroClamp = 1000;
struct ZeroBias {
    half2_t lo, hi;
    int zc;       // the clamped zero point the biases encode
};
__device__ __forceinline__ ZeroBias zero_bias(int z) {
    const int zc = min(max(z, -kZeroClamp), kZeroClamp);
    const _Float16 zh = (_Float16)zc;                       // exact
    const _Float16 lo = (_Float16)-1024.0f - zh, hi = (_Float16)-64.0f - zh;
    return ZeroBias{(half2_t){lo, lo}, (half2_t){hi, hi}, zc};
}
__device__ __forceinline__ void codes_word_zp(uint32_t w, const CodeConsts& k, const ZeroBias& b,
                                              half2_t (&q)[4]) {
    const half2_t inv16 = {(_Float16)0.0625f, (_Float16)0.0625f};
    const uint32_t w8 = w >> 8;
    q[0] = as_h2((w & k.m_lo) | k.magic) + b.lo;
    q[1] = __builtin_elementwise_fma(as_h2((w & k.m_hi) | k.magic), inv16, b.hi);
    q[2] = as_h2((w8 & k.m_lo) | k.magic) + b.lo;
    q[3] = __builtin_elementwise_fma(as_h2((w8 & k.m_hi) | k.magic), inv16, b.hi);
}

// acc += sum of the word's 8 products q*x (paired activations xp), each
// product exact in fp32 (v_dot2_f32_f16), so the rounding error of the
// accumulation is relative to sum |q x|.
__device__ __forceinline__ float dot_word(uint32_t w, const uint4& xp, float acc,
                                          const CodeConsts& k) {
    half2_t q[4];
    codes_word(w, k, q);
    acc = __builtin_amdgcn_fdot2(q[0], as_h2(xp.x), acc, false);
    acc = __builtin_amdgcn_fdot2(q[1], as_h2(xp.y), acc, false);
    acc = __builtin_amdgcn_fdot2(q[2], as_h2(xp.z), acc, false);
    acc = __builtin_amdgcn_fdot2(q[3], as_h2(xp.w), acc, false);
    return acc;
}

// Lanes of a wave that share one weight row in the M = 1 GEMV (the
// persistent kernel and the dependent-sequence kernel use the same split, so
// their sums are taken in the same order): 64, unless the row's K/32 chunks
// are a multiple of 16 but not of 64 and the matrix has at least 128 rows
// per compute unit, then 16 (four rows side by side, so no lane idles in a
// row's last step; with fewer rows the 8-row groups would leave waves idle).
__host__ __device__ inline int gemv_lanes_per_row(int64_t K, int64_t N, int num_cu) {
    const int64_t chunks = K / 32;
    return (chunks % 64 != 0 && chunks % 16 == 0 && N >= (int64_t)128 * num_cu) ? 16 : 64;
}

// Raw buffer resource over [base, base + bytes) for gfx9 (data format 32;
// reads past `bytes` return 0 instead of touching memory).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint64_t bytes) {
    const int n = bytes > 0xFFFFFFFFull ? (int)0xFFFFFFFFu : (int)(uint32_t)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, n, 0x00020000);
}

// One packed word -> its 8 dequantized weights fp16(s*q) as 4 half2 in the
// paired order (w0,w4),(w1,w5),(w2,w6),(w3,w7): exact codes (codes_word)
// times the scale, rounded once to nearest even.
__device__ __forceinline__ void dequant_word(uint32_t w, half2_t s2, half2_t (&out)[4],
                                             const CodeConsts& k) {
    half2_t q[4];
    codes_word(w, k, q);
    out[0] = q[0] * s2;
    out[1] = q[1] * s2;
    out[2] = q[2] * s2;
    out[3] = q[3] * s2;
}

// Cache policy of the weight stream: non-temporal (the loads' slc/nt bit).
constexpr int kStreamLoad = 2;

// Sum over the 64 lanes with DPP row operations (gfx9 wave64 pattern):
// butterflies inside quads, mirrors inside 16-lane rows, then row broadcasts
// 15 and 31.  The total ends in lane 63.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_add(float v) {
    const int moved = __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xF, false);
    return v + __int_as_float(moved);
}
__device__ __forceinline__ float wave_sum_lane63(float v) {
    v = dpp_add<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
    v = dpp_add<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
    v = dpp_add<0x141, 0xF>(v);  // row_half_mirror
    v = dpp_add<0x140, 0xF>(v);  // row_mirror: every lane holds its row's sum
    v = dpp_add<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
    v = dpp_add<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
    return v;
}
// Sum over each 16-lane row (the first four steps above): every lane of a
// row holds its row's total.
__device__ __forceinline__ float row16_sum(float v) {
    v = dpp_add<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
    v = dpp_add<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
    v = dpp_add<0x141, 0xF>(v);  // row_half_mirror
    v = dpp_add<0x140, 0xF>(v);  // row_mirror
    return v;
}

}  // namespace w4a16

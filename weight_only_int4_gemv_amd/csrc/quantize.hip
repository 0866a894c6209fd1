// quantize.hip — RTN INT4 quantizers (symmetric, and asymmetric with a zero
// point per group), one fp16 scale per group of
// G elements along K (G = 128 by default; 32, 64 and 256 as in [QUANT]'s
// granularity table and GPTQ group_size table), packed eight codes per
// uint32 ([QUANT] sub-section 2 equations, sub-section 3 per-group listing;
// [INT4] INT4 paragraph).
//
// Work split: G/8 consecutive lanes of a wave per (row, group).  Each lane
// loads 16 bytes (8 fp16), the lanes reduce the absolute maximum (the
// asymmetric quantizer: the maximum and the minimum) with DPP (and one
// cross-row swap for G = 256), and each lane writes the one packed word its
// 8 elements form; the group's lanes write its G/2 contiguous bytes.  HBM
// traffic per element: 2 B in, 0.5 + 2/G B out (0.5 + 4/G with zero points).
//
// Bit-exactness:
//   - |w| is compared as the integer w & 0x7FFF (order of finite fp16
//     magnitudes is the order of their bit patterns);
//   - s = fp16_rne(a / 7), formed as fp16_rne(a * fp32(1/7)): for every
//     finite fp16 a the two agree (checked over all 31,743 positive finite
//     values, and 0, infinity and NaN map alike), so the scale needs one
//     multiply instead of an IEEE division;
//   - q = clamp(rint(w / s), -8, 7) with rint (half to even) of the quotient
//     rounded to fp32: for fp16 w and s a non-tie quotient is at least 2^-15
//     (relative) away from a tie, so the fp32 quotient rounds to the same
//     integer as the exact one.  The code plus 8 is first formed as
//     u = fma(w, rcp(s), 8) (v_rcp_f32, relative error below 2^-22;
//     |w / s| <= 7.004, or < 10.5 when s is an fp16 subnormal, so w * rcp(s)
//     is within 3e-6 of w / s, and the fma's one rounding of a value below
//     32 adds at most 2^-20): u is within 4e-6 of w / s + 8, and rint(u) -
//     8 can differ from rint(w / s) only if u lies within 4e-6 of a
//     half-integer (8 is even, so away from ties the shift commutes with
//     rounding); a lane that sees a u within 2e-5 of one (about 2 in 10^5
//     elements of Gaussian weights, and every exact tie) redoes its 8
//     elements with the IEEE fp32 division.
#include <atomic>

#include "w4a16_device.h"
#include "w4a16_launch.h"

namespace w4a16 {

namespace {
// Group quantizer launch: U groups per lane slice and step, and at most this
// many resident 256-thread blocks per compute unit (the grid walks the rest).
constexpr int kQuantizeGroupsPerStep = 2;
constexpr int kQuantizeBlocksPerCu = 8;

// max over the 16 lanes of a DPP row (quad butterflies, then half-row and
// row mirrors); every lane of the row receives it.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_max(uint32_t v) {
    return max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false));
}
// max over the LG lanes of a group (LG = 4, 8, 16 or 32 consecutive lanes);
// every lane of the group receives it.  Quad butterflies, then the half-row
// and row mirrors (each lane meets the lane its mirror maps it to, which
// after the quad step carries that quad's maximum), then a swap of the two
// 16-lane rows of a 32-lane group.
template <int LG>
__device__ __forceinline__ uint32_t group_max(uint32_t v) {
    static_assert(LG == 4 || LG == 8 || LG == 16 || LG == 32, "lanes per group");
    v = dpp_max<0xB1>(v);                                   // quad_perm [1,0,3,2]
    v = dpp_max<0x4E>(v);                                   // quad_perm [2,3,0,1]
    if constexpr (LG >= 8) v = dpp_max<0x141>(v);           // row_half_mirror
    if constexpr (LG >= 16) v = dpp_max<0x140>(v);          // row_mirror
    if constexpr (LG == 32) v = max(v, (uint32_t)__shfl_xor((int)v, 16));
    return v;
}

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef short i16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ u16x2 as_u16x2(uint32_t w) { return __builtin_bit_cast(u16x2, w); }

// |w| of the 8 fp16 values of a lane, as the largest magnitude bit pattern
// (sign bits cleared, then 16-bit maxima two at a time).
__device__ __forceinline__ uint32_t absmax8(const uint4& v) {
    const u16x2 a = as_u16x2(v.x & 0x7FFF7FFFu), b = as_u16x2(v.y & 0x7FFF7FFFu);
    const u16x2 c = as_u16x2(v.z & 0x7FFF7FFFu), d = as_u16x2(v.w & 0x7FFF7FFFu);
    const u16x2 m = __builtin_elementwise_max(__builtin_elementwise_max(a, b),
                                              __builtin_elementwise_max(c, d));
    return max((uint32_t)m.x, (uint32_t)m.y);
}

// Packed word of 8 codes, each an integer-valued float in [0, 15]: codes
// 0, 2, 4, 6 in the bytes of one word, 1, 3, 5, 7 in another, then the
// second shifted into the high nibbles (element i at bits 4i).
__device__ __forceinline__ uint32_t pack_codes8(const float (&c)[8]) {
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        lo = __builtin_amdgcn_cvt_pk_u8_f32(c[2 * j], j, lo);
        hi = __builtin_amdgcn_cvt_pk_u8_f32(c[2 * j + 1], j, hi);
    }
    return lo | (hi << 4);
}

// Scale bits of a group (or row) whose absolute maximum has bit pattern m.
__device__ __forceinline__ uint16_t scale_of_absmax(uint32_t m) {
    const float a = f16_bits_to_f32((uint16_t)m);
    constexpr float kSeventh = 1.0f / 7.0f;   // 2^(4-1) - 1 = 7; fp32(1/7)
    return f32_to_f16_bits(a * kSeventh);     // = fp16_rne(a / 7), see above
}

__device__ __forceinline__ uint32_t codes8(const uint4& v, uint16_t s_bits);

// One lane's 8 elements of a group -> its packed word, and the group scale.
template <int LG>
__device__ __forceinline__ uint32_t quantize8(const uint4& v, uint16_t& s_bits) {
    s_bits = scale_of_absmax(group_max<LG>(absmax8(v)));
    return codes8(v, s_bits);
}

// The packed word of 8 elements against the scale with bits s_bits.
__device__ __forceinline__ uint32_t codes8(const uint4& v, uint16_t s_bits) {
    const float s = f16_bits_to_f32(s_bits);
    if (s == 0.0f) return 0x88888888u;   // every code 0 (all lanes of the group alike)
    const uint32_t h[4] = {v.x, v.y, v.z, v.w};
    const float inv = __builtin_amdgcn_rcpf(s);
    float c[8];
    float dist = 0.0f;                         // largest |u - rint(u)| of the 8
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float w = f16_bits_to_f32((uint16_t)(h[i >> 1] >> (16 * (i & 1))));
        const float u = fmaf(w, inv, 8.0f);       // w / s + 8, within 4e-6
        const float r = rintf(u);
        dist = fmaxf(dist, fabsf(u - r));
        // code = clamp(rint(w / s), -8, 7) + 8 = clamp(r, 0, 15), exact in fp32
        c[i] = __builtin_amdgcn_fmed3f(r, 0.0f, 15.0f);
    }
    if (dist > 0.49998f) {                     // a half-integer within 2e-5: redo exactly
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float w = f16_bits_to_f32((uint16_t)(h[i >> 1] >> (16 * (i & 1))));
            c[i] = fminf(fmaxf(rintf(w / s), -8.0f), 7.0f) + 8.0f;
        }
    }
    return pack_codes8(c);
}

// ---- asymmetric INT4 ([QUANT] sub-section 2, asymmetric equations) ----
//   s = fp16_rne((max - min) / 15), z = -rint(min / s), q = clamp(rint(w / s)
//   + z, 0, 15), stored as the nibble q itself; s = 0 (a group whose range
//   rounds to 0) stores z = 0 and q = 0.
// Bit-exactness:
//   - the scale in binary64: max - min of two fp16 values is exact (at most
//     40 significant bits); the IEEE division by 15 and the rounding to fp16
//     below give the RNE of the exact quotient: (max - min) / 15 is either
//     dyadic (then exact in binary64) or has the period-4 binary expansion
//     of 1/15, which never puts a 53-bit rounding on a fp16 tie;
//   - a quotient a / s of two fp16 values that is not a tie lies at least
//     2^-13 from one (write a = A 2^e, s = B 2^f with 11-bit integers A, B:
//     the distance is a nonzero multiple of 2^(e-f) / (2B), and where it
//     matters, |a / s| >= 1/2, 2^(e-f) >= B / (2A)), and |min / s|, |w / s|
//     stay below 2^15 (the range is at least one fp16 spacing of min);
//   - 1/s is formed as r = rcp_f32(s) (relative error below 2^-22) refined
//     by one binary64 Newton step (relative error below 2^-43);
//   - z: p = min * r is within 2^-27 of min / s; rint(p) is z unless p lies
//     within 2^-20 of a half-integer (exact ties only), where the IEEE
//     division decides;
//   - codes in fp32: r is split into r_hi = fp32(r) and r_lo = fp32(r -
//     r_hi), and u = fma(w, r_lo, fma(w, r_hi, z)).  Where |w / s + z| < 15.99
//     (every code the clamp does not fix), each fma rounds a value below 16
//     (error at most 2^-21) and r_hi + r_lo misses 1/s by under 2^-43
//     relative (2^-27 absolute on w / s), so u is within 2^-19.9 of w / s
//     + z.  rint(u) then equals rint(w / s + z) = rint(w / s) + z unless u is
//     within 2^-15 of a half-integer, where the lane redoes its 8 elements
//     with the binary64 division (exact ties among them: rint(w / s) + z
//     differs from rint(w / s + z) at a tie when z is odd).  Beyond 16 in
//     magnitude the clamp gives 0 or 15 whatever the rounding.

// fp16 bits of the round-to-nearest-even of v (0 <= v < 65520): the integer
// rint(v / u) times the fp16 spacing u = 2^(e - 10) at v's binade (2^-24
// below 2^-14), both scalings by powers of two exact.
__device__ __forceinline__ uint16_t f16_rne_from_f64(double v) {
    if (v == 0.0) return 0;
    const uint64_t b = (uint64_t)__double_as_longlong(v);
    int e = (int)((b >> 52) & 0x7FF) - 1023;      // v > 0 is a normal binary64
    if (e < -14) e = -14;
    const double m = rint(ldexp(v, 10 - e));      // at most 2^11
    return f32_to_f16_bits((float)ldexp(m, e - 10));
}

// Order-preserving key of a finite fp16 bit pattern h (sign-magnitude to
// offset binary, -0 just below +0): h ^ 0xFFFF when the sign bit is set,
// else h ^ 0x8000 (formed two at a time below).  Its inverse:
__device__ __forceinline__ uint32_t f16_from_key(uint32_t k) {
    return k ^ ((k & 0x8000u) ? 0x8000u : 0xFFFFu);
}

// Largest key and largest 0xFFFF - key of a lane's 8 values (the maximum
// and, complemented, the minimum), two 16-bit keys at a time: a negative
// half (sign bit set) has all bits flipped, a positive one its sign bit set.
__device__ __forceinline__ void minmax_keys8(const uint4& v, uint32_t& kmax, uint32_t& kmin_c) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    u16x2 hi, lo;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const i16x2 sgn = __builtin_bit_cast(i16x2, w[i]) >> (short)15;      // 0 or -1 per half
        const u16x2 key = as_u16x2(w[i] ^ (__builtin_bit_cast(uint32_t, sgn) | 0x80008000u));
        hi = i == 0 ? key : __builtin_elementwise_max(hi, key);
        lo = i == 0 ? key : __builtin_elementwise_min(lo, key);
    }
    kmax = max((uint32_t)hi.x, (uint32_t)hi.y);
    kmin_c = 0xFFFFu - min((uint32_t)lo.x, (uint32_t)lo.y);
}

// 1/s to within 2^-43 (relative) for an fp16 scale s > 0: the fp32
// reciprocal (relative error below 2^-22) and one binary64 Newton step.
__device__ __forceinline__ double recip_of_scale(double s) {
    const double r0 = (double)__builtin_amdgcn_rcpf((float)s);
    return fma(r0, fma(-s, r0, 1.0), r0);
}

// What the codes of a group need: the scale (binary64 and fp16 bits), 1/s
// split in two fp32 parts, and the zero point.
struct AsymCode {
    double s;
    float r_hi, r_lo, zf;
    int16_t zero;
    uint16_t s_bits;
};
__device__ __forceinline__ AsymCode asym_code(uint16_t s_bits, int16_t zero, double r) {
    AsymCode c;
    c.s = (double)f16_bits_to_f32(s_bits);
    c.s_bits = s_bits;
    c.zero = zero;
    c.r_hi = (float)r;
    c.r_lo = (float)(r - (double)c.r_hi);
    c.zf = (float)zero;
    return c;
}
// ... for a stored scale and zero point
__device__ __forceinline__ AsymCode asym_code(uint16_t s_bits, int16_t zero) {
    const double s = (double)f16_bits_to_f32(s_bits);
    return asym_code(s_bits, zero, s == 0.0 ? 0.0 : recip_of_scale(s));
}

// Scale, zero point (and reciprocal) of a group (or row) from its reduced
// keys.
__device__ __forceinline__ AsymCode asym_params(uint32_t kmax, uint32_t kmin_c) {
    const double mx = (double)f16_bits_to_f32((uint16_t)f16_from_key(kmax));
    const double mn = (double)f16_bits_to_f32((uint16_t)f16_from_key(0xFFFFu - kmin_c));
    const uint16_t s_bits = f16_rne_from_f64((mx - mn) / 15.0);   // 2^4 - 1 = 15
    const double s = (double)f16_bits_to_f32(s_bits);
    if (s == 0.0) return asym_code(s_bits, 0, 0.0);
    const double r = recip_of_scale(s);
    const double p = mn * r;
    double q = rint(p);
    if (fabs(p - q) > 0.5 - 0x1p-20) q = rint(mn / s);   // a tie: the division decides
    return asym_code(s_bits, (int16_t)(int)-q, r);
}

// The packed word of 8 elements against a group's scale and zero point.
__device__ __forceinline__ uint32_t codes8_asym(const uint4& v, const AsymCode& p) {
    if (p.s == 0.0) return 0u;                           // every code 0
    const uint32_t h[8] = {v.x & 0xFFFFu, v.x >> 16, v.y & 0xFFFFu, v.y >> 16,
                           v.z & 0xFFFFu, v.z >> 16, v.w & 0xFFFFu, v.w >> 16};
    float c[8];
    float dist = 0.0f;                                   // largest |u - rint(u)|
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float w = f16_bits_to_f32((uint16_t)h[i]);
        const float u = fmaf(w, p.r_lo, fmaf(w, p.r_hi, p.zf));   // w / s + z, within 2^-19.9
        const float q = rintf(u);
        dist = fmaxf(dist, fabsf(u - q));
        c[i] = __builtin_amdgcn_fmed3f(q, 0.0f, 15.0f);
    }
    if (dist > 0.5f - 0x1p-15f) {                        // near a half-integer: redo exactly
        const double z = (double)p.zero;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const double q = rint((double)f16_bits_to_f32((uint16_t)h[i]) / p.s);
            c[i] = (float)fmin(fmax(q + z, 0.0), 15.0);
        }
    }
    return pack_codes8(c);
}

// EPL elements of a lane (EPL / 8 vectors, all of one group) -> their packed
// words, and the group's scale and zero point.
template <int LG, int EPL>
__device__ __forceinline__ void quantize_asym(const uint4 (&v)[EPL / 8], uint32_t (&words)[EPL / 8],
                                              uint16_t& s_bits, int16_t& zero) {
    uint32_t kmax = 0, kmin_c = 0;
#pragma unroll
    for (int i = 0; i < EPL / 8; ++i) {
        uint32_t a, b;
        minmax_keys8(v[i], a, b);
        kmax = max(kmax, a);
        kmin_c = max(kmin_c, b);
    }
    const AsymCode p = asym_params(group_max<LG>(kmax), group_max<LG>(kmin_c));
    s_bits = p.s_bits;
    zero = p.zero;
#pragma unroll
    for (int i = 0; i < EPL / 8; ++i) words[i] = codes8_asym(v[i], p);
}

}  // namespace

// Each LG-lane slice of a wave quantizes U groups per step (groups g, g +
// stride, ..., stride = the slices in the grid); the grid is a few blocks
// per compute unit and walks the groups in steps of U * stride.  The loads
// of step t + 1 are issued before step t is quantized (two register sets,
// the loop unrolled over two steps), and every load is unconditional (a
// group past the end reloads the last group and stores nothing), so the
// compiler's counter wait before step t covers exactly step t's loads.  All
// LG lanes of a slice share g, so the reductions only ever combine lanes
// that are active together.
//
// perm (act-order layout, [QUANT] GPTQ section: columns quantized and stored
// in the order perm): NULL, or device int32 [K]; column j of the output is
// column perm[j] of W (an index outside [0, K) reads as 0), gathered with
// 2-byte loads instead of one 16-byte load per lane (PERM: a copy of the
// kernel of its own; the gather's loads depend on the perm loads, so its
// steps do not overlap).
//
// ASYM: the asymmetric quantizer, which also writes one int16 zero point per
// group to `zeros` (laid out like the scales).
template <int LG, int U, bool ASYM, bool PERM, int EPL>
__global__ __launch_bounds__(256) void quantize_kernel(const uint4* __restrict__ W,
                                                       uint32_t* __restrict__ packed,
                                                       uint16_t* __restrict__ scales,
                                                       int16_t* __restrict__ zeros,
                                                       int64_t total_groups, int K,
                                                       const int* __restrict__ perm) {
    static_assert(EPL == 8 || (EPL == 16 && ASYM && !PERM), "elements per lane");
    constexpr int V = EPL / 8;                           // 16-byte vectors per lane and group
    constexpr int GV = LG * V;                           // vectors (and packed words) per group
    typedef unsigned v4u __attribute__((ext_vector_type(4)));
    const int lg = threadIdx.x & (LG - 1);              // lane within the group
    const int64_t stride = (int64_t)gridDim.x * (blockDim.x / LG);
    const int64_t step = (int64_t)U * stride;
    const v4u* Wv = reinterpret_cast<const v4u*>(W);

    // vector i of a lane is vector i * LG + lg of its group (contiguous over
    // the group's lanes for each i)
    auto load = [&](v4u (&a)[U][V], int64_t g) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t gu = min(g + u * stride, total_groups - 1);
            if constexpr (!PERM) {
#pragma unroll
                for (int i = 0; i < V; ++i)   // W is read once
                    a[u][i] = __builtin_nontemporal_load(Wv + gu * GV + i * LG + lg);
            } else {
                const int64_t gpr = K / (LG * 8);                // groups per row
                const int64_t n = gu / gpr;
                const int col = (int)(gu - n * gpr) * (LG * 8) + lg * 8;
                const uint16_t* row = reinterpret_cast<const uint16_t*>(W) + n * K;
                uint32_t h[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int p = perm[col + i];
                    h[i] = (uint32_t)p < (uint32_t)K ? row[p] : 0u;
                }
                a[u][0] = (v4u){h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                                h[6] | (h[7] << 16)};
            }
        }
    };
    auto work = [&](const v4u (&a)[U][V], int64_t g) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t gu = g + u * stride;
            if (gu < total_groups) {
                uint4 v[V];
#pragma unroll
                for (int i = 0; i < V; ++i) v[i] = make_uint4(a[u][i].x, a[u][i].y, a[u][i].z, a[u][i].w);
                uint16_t sb;
                if constexpr (ASYM) {
                    int16_t zb;
                    uint32_t words[V];
                    quantize_asym<LG, EPL>(v, words, sb, zb);
#pragma unroll
                    for (int i = 0; i < V; ++i) packed[gu * GV + i * LG + lg] = words[i];
                    if (lg == 0) {
                        scales[gu] = sb;
                        zeros[gu] = zb;
                    }
                } else {
                    packed[gu * LG + lg] = quantize8<LG>(v[0], sb);
                    if (lg == 0) scales[gu] = sb;
                }
            }
        }
    };

    const int64_t g0 = (int64_t)blockIdx.x * (blockDim.x / LG) + (threadIdx.x / LG);
    v4u a[U][V], b[U][V];
    load(a, g0);
    for (int64_t g = g0; g < total_groups; g += 2 * step) {
        load(b, g + step);
        work(a, g);
        load(a, g + 2 * step);
        work(b, g + step);
    }
}

// Q4_0 blocks ([QUANT] GGUF section, Q4_0: 32 elements in 18 bytes, the
// fp16 scale d then 16 code bytes with element 2i in the low nibble of byte
// 2+i): the symmetric quantizer on groups of 32 (four lanes per block, as
// for G = 32), each lane storing its packed word at byte 2 + 4*lane of the
// block as two 16-bit halves (blocks are only 2-byte aligned) and the
// block's first lane storing d.
// ---- per-channel scales ([QUANT] sub-section 3 granularity table, per
// channel: one scale per output row; the GPTQ section's group_size -1):
// the group is the whole row.  One kernel reduces each row (absolute maximum,
// or maximum and minimum keys) to its scale (and zero point); a second forms
// the codes against it with the same per-element arithmetic as the group
// quantizer, so both give the bits the group formulas give with G = K.

// The 8 elements of row `row` at columns c0 .. c0+7 of the stored order
// (W's own columns, or W[:, perm[...]] with an index outside [0, K) read as 0).
__device__ __forceinline__ uint4 row_load8(const uint16_t* __restrict__ row, int c0, int K,
                                           const int* __restrict__ perm) {
    if (perm == nullptr) return *reinterpret_cast<const uint4*>(row + c0);
    uint32_t h[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int p = perm[c0 + i];
        h[i] = (uint32_t)p < (uint32_t)K ? row[p] : 0u;
    }
    return make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                      h[6] | (h[7] << 16));
}

// max over the 64 lanes of the wave (every lane receives it)
__device__ __forceinline__ uint32_t wave_max64(uint32_t v) {
    v = group_max<32>(v);
    return max(v, (uint32_t)__shfl_xor((int)v, 32));
}

template <bool ASYM>
__global__ __launch_bounds__(256) void row_scale_kernel(const uint16_t* __restrict__ W,
                                                        int64_t N, int K,
                                                        uint16_t* __restrict__ scales,
                                                        int16_t* __restrict__ zeros,
                                                        const int* __restrict__ perm) {
    __shared__ uint32_t red[2][4];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int chunks = K >> 3;
    for (int64_t n = blockIdx.x; n < N; n += gridDim.x) {
        const uint16_t* row = W + n * (int64_t)K;
        uint32_t a = 0, b = 0;           // absmax; or max key, max complemented key
        for (int c = threadIdx.x; c < chunks; c += blockDim.x) {
            const uint4 v = row_load8(row, c * 8, K, perm);
            if constexpr (ASYM) {
                uint32_t ka, kb;
                minmax_keys8(v, ka, kb);
                a = max(a, ka);
                b = max(b, kb);
            } else {
                a = max(a, absmax8(v));
            }
        }
        a = wave_max64(a);
        if constexpr (ASYM) b = wave_max64(b);
        if (lane == 0) {
            red[0][wave] = a;
            red[1][wave] = b;
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            a = max(max(red[0][0], red[0][1]), max(red[0][2], red[0][3]));
            if constexpr (ASYM) {
                b = max(max(red[1][0], red[1][1]), max(red[1][2], red[1][3]));
                const AsymCode p = asym_params(a, b);
                scales[n] = p.s_bits;
                zeros[n] = p.zero;
            } else {
                scales[n] = scale_of_absmax(a);
            }
        }
        __syncthreads();                 // red is reused by the next row
    }
}

template <bool ASYM>
__global__ __launch_bounds__(256) void row_codes_kernel(const uint16_t* __restrict__ W,
                                                        int64_t N, int K,
                                                        uint32_t* __restrict__ packed,
                                                        const uint16_t* __restrict__ scales,
                                                        const int16_t* __restrict__ zeros,
                                                        const int* __restrict__ perm) {
    const int wpr = K >> 3;              // packed words per row
    const int64_t words = N * (int64_t)wpr;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < words;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t n = i / wpr;
        const int c = (int)(i - n * wpr);
        const uint4 v = row_load8(W + n * (int64_t)K, c * 8, K, perm);
        packed[i] = ASYM ? codes8_asym(v, asym_code(scales[n], zeros[n])) : codes8(v, scales[n]);
    }
}

// One pass for rows of up to 256 * CPT chunks: every thread keeps its
// chunks of the row (c = thread + 256 i) in registers, the block reduces them
// to the row's scale (and zero point), and each thread then forms the codes
// of the chunks it holds, so W is read once where the two kernels above read
// it twice.  The reduction, the scale and the codes are those functions'
// own, so the bits are the same.
template <bool ASYM, int CPT>
__global__ __launch_bounds__(256) void row_quantize_kernel(const uint16_t* __restrict__ W,
                                                           int64_t N, int K,
                                                           uint32_t* __restrict__ packed,
                                                           uint16_t* __restrict__ scales,
                                                           int16_t* __restrict__ zeros,
                                                           const int* __restrict__ perm) {
    __shared__ uint32_t red[2][4];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int chunks = K >> 3;
    for (int64_t n = blockIdx.x; n < N; n += gridDim.x) {
        const uint16_t* row = W + n * (int64_t)K;
        uint4 v[CPT];
        uint32_t a = 0, b = 0;           // absmax; or max key, max complemented key
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int c = (int)threadIdx.x + i * 256;
            v[i] = make_uint4(0, 0, 0, 0);
            if (c < chunks) {
                v[i] = row_load8(row, c * 8, K, perm);
                if constexpr (ASYM) {
                    uint32_t ka, kb;
                    minmax_keys8(v[i], ka, kb);
                    a = max(a, ka);
                    b = max(b, kb);
                } else {
                    a = max(a, absmax8(v[i]));
                }
            }
        }
        a = wave_max64(a);
        if constexpr (ASYM) b = wave_max64(b);
        if (lane == 0) {
            red[0][wave] = a;
            red[1][wave] = b;
        }
        __syncthreads();
        a = max(max(red[0][0], red[0][1]), max(red[0][2], red[0][3]));
        if constexpr (ASYM) b = max(max(red[1][0], red[1][1]), max(red[1][2], red[1][3]));
        __syncthreads();                 // red is reused by the next row
        uint32_t* const prow = packed + n * (int64_t)chunks;
        if constexpr (ASYM) {
            const AsymCode p = asym_params(a, b);
            if (threadIdx.x == 0) {
                scales[n] = p.s_bits;
                zeros[n] = p.zero;
            }
#pragma unroll
            for (int i = 0; i < CPT; ++i) {
                const int c = (int)threadIdx.x + i * 256;
                if (c < chunks) prow[c] = codes8_asym(v[i], p);
            }
        } else {
            const uint16_t sb = scale_of_absmax(a);
            if (threadIdx.x == 0) scales[n] = sb;
#pragma unroll
            for (int i = 0; i < CPT; ++i) {
                const int c = (int)threadIdx.x + i * 256;
                if (c < chunks) prow[c] = codes8(v[i], sb);
            }
        }
    }
}

template <bool ASYM>
hipError_t launch_quantize_rows(const uint16_t* W, int64_t N, int64_t K, uint32_t* packed,
                                uint16_t* scales, int16_t* zeros, const int* perm,
                                hipStream_t stream) {
    // one block per row (the grid walks the rest past 2^20 rows)
    const int64_t chunks = K / 8;
    const unsigned rblocks = (unsigned)(N < ((int64_t)1 << 20) ? N : ((int64_t)1 << 20));
#define W4A16_ROWS(CPT)                                                                     \
    hipLaunchKernelGGL((row_quantize_kernel<ASYM, CPT>), dim3(rblocks), dim3(256), 0, stream, \
                       W, N, (int)K, packed, scales, zeros, perm);                          \
    return hipGetLastError()
    if (chunks <= 256 * 4) { W4A16_ROWS(4); }
    if (chunks <= 256 * 8) { W4A16_ROWS(8); }
    if (chunks <= 256 * 16) { W4A16_ROWS(16); }
#undef W4A16_ROWS
    // longer rows: the row reduction, then the codes
    const int64_t sblocks = N < 4096 ? N : 4096;
    hipLaunchKernelGGL((row_scale_kernel<ASYM>), dim3((unsigned)sblocks), dim3(256), 0, stream,
                       W, N, (int)K, scales, zeros, perm);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t words = N * (K / 8);
    int64_t cblocks = (words + 255) / 256;
    if (cblocks > 16384) cblocks = 16384;
    hipLaunchKernelGGL((row_codes_kernel<ASYM>), dim3((unsigned)cblocks), dim3(256), 0, stream,
                       W, N, (int)K, packed, scales, zeros, perm);
    return hipGetLastError();
}

template <int U>
__global__ __launch_bounds__(256) void quantize_q4_0_kernel(const uint4* __restrict__ W,
                                                            uint16_t* __restrict__ blocks,
                                                            int64_t total_blocks) {
    constexpr int LG = 4;
    const int lg = threadIdx.x & (LG - 1);
    const int64_t stride = (int64_t)gridDim.x * (blockDim.x / LG);
    typedef unsigned v4u __attribute__((ext_vector_type(4)));
    const v4u* Wv = reinterpret_cast<const v4u*>(W);
    for (int64_t g = (int64_t)blockIdx.x * (blockDim.x / LG) + (threadIdx.x / LG);
         g < total_blocks; g += U * stride) {
        v4u a[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t gu = g + u * stride;
            a[u] = gu < total_blocks ? __builtin_nontemporal_load(Wv + gu * LG + lg)
                                     : (v4u){0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t gu = g + u * stride;
            if (gu < total_blocks) {
                uint16_t d;
                const uint32_t word = quantize8<LG>(make_uint4(a[u].x, a[u].y, a[u].z, a[u].w), d);
                uint16_t* blk = blocks + gu * 9;             // 18 bytes = 9 halves
                blk[1 + 2 * lg] = (uint16_t)(word & 0xFFFFu);
                blk[2 + 2 * lg] = (uint16_t)(word >> 16);
                if (lg == 0) blk[0] = d;
            }
        }
    }
}

hipError_t launch_quantize_q4_0(const uint16_t* W, int64_t N, int64_t K, uint8_t* blocks,
                                hipStream_t stream) {
    const int64_t total = N * (K / 32);
    if (total == 0) return hipSuccess;
    constexpr int U = 2, per_block = 256 / 4;
    int64_t grid = (total + per_block * U - 1) / (per_block * U);
    if (grid > 65536) grid = 65536;
    hipLaunchKernelGGL((quantize_q4_0_kernel<U>), dim3((unsigned)grid), dim3(256), 0, stream,
                       reinterpret_cast<const uint4*>(W), reinterpret_cast<uint16_t*>(blocks),
                       total);
    return hipGetLastError();
}

// LG: lanes per group; EPL: elements per lane (G = LG * EPL); EPL = 16 only
// for the asymmetric quantizer without perm, whose per-group scale, zero
// point and reciprocal then serve 16 elements of each lane instead of 8.
template <int LG, int U, int EPL = 8>
hipError_t launch_quantize_t(const uint16_t* W, int64_t groups, int64_t K, const int* perm,
                             uint32_t* packed, uint16_t* scales, int16_t* zeros,
                             hipStream_t stream, int num_cu) {
    constexpr int per_block = 256 / LG;                  // groups per block and step
    const int64_t need = (groups + per_block * U - 1) / (per_block * U);
    const uint4* Wv = reinterpret_cast<const uint4*>(W);
    // one resident round of blocks (the occupancy query's count per CU, at
    // most kQuantizeBlocksPerCu), walking the groups in grid strides
#define W4A16_QUANTIZE(ASYM, PERM, E)                                                             \
    do {                                                                                          \
        auto kern = quantize_kernel<LG, U, ASYM, PERM, E>;                                        \
        static std::atomic<int> resident{0};                                                      \
        int r = resident.load(std::memory_order_relaxed);                                         \
        if (r == 0) {                                                                             \
            const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(                    \
                &r, reinterpret_cast<const void*>(kern), 256, 0);                                 \
            if (e != hipSuccess) return e;                                                        \
            r = r < 1 ? 1 : (r > kQuantizeBlocksPerCu ? kQuantizeBlocksPerCu : r);                \
            resident.store(r, std::memory_order_relaxed);                                         \
        }                                                                                         \
        const int64_t cap = (int64_t)num_cu * r;                                                  \
        const int64_t blocks = need < cap ? need : cap;                                           \
        hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(256), 0, stream, Wv, packed, scales, \
                           zeros, groups, (int)K, perm);                                          \
    } while (0)
    if constexpr (EPL == 16) {
        W4A16_QUANTIZE(true, false, 16);
    } else if (zeros != nullptr) {
        if (perm != nullptr) W4A16_QUANTIZE(true, true, 8);
        else W4A16_QUANTIZE(true, false, 8);
    } else {
        if (perm != nullptr) W4A16_QUANTIZE(false, true, 8);
        else W4A16_QUANTIZE(false, false, 8);
    }
#undef W4A16_QUANTIZE
    return hipGetLastError();
}

// Weights in their own column order, on a flat grid: a slot is EPL
// consecutive elements (EPL / 8 chunks of 8) of one group; block b takes the
// slots [b 256 CPT, (b + 1) 256 CPT) (thread t the slots t + 256 i), issues
// all their loads first and then quantizes them, LG lanes a group with the
// per-lane arithmetic of quantize_kernel (a group never straddles a block:
// 256 is a multiple of LG, and groups never straddle rows).  Measured against
// the persistent quantize_kernel (bit-identical): symmetric (CPT 2)
// 28672x8192 106-109 against 112-116 us, 14336x4096 27.0-27.5 against
// 30.2-31.7 us at every group size; asymmetric (CPT 1, 16 elements a lane
// from group 64 up) 14336x4096 31.0-32.3 against 37.6-38.7 us from group 64
// up, 40.5-40.9 against 47.0 us at group 32, 28672x8192 115-118 against
// 131-137 us.
template <int LG, int CPT, bool ASYM, int EPL>
__global__ __launch_bounds__(256) void quantize_flat_kernel(const uint4* __restrict__ W,
                                                            int64_t slots,
                                                            uint32_t* __restrict__ packed,
                                                            uint16_t* __restrict__ scales,
                                                            int16_t* __restrict__ zeros) {
    static_assert(EPL == 8 || (EPL == 16 && ASYM), "elements per lane");
    constexpr int V = EPL / 8;
    const int64_t base = (int64_t)blockIdx.x * (256 * CPT) + threadIdx.x;
    uint4 v[CPT][V];
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
        const int64_t e = base + (int64_t)i * 256;
#pragma unroll
        for (int k = 0; k < V; ++k)
            v[i][k] = e < slots ? W[e * V + k] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
        const int64_t e = base + (int64_t)i * 256;
        // every lane takes part in the group reductions
        uint32_t words[V];
        uint16_t sb;
        int16_t z = 0;
        if constexpr (ASYM)
            quantize_asym<LG, EPL>(v[i], words, sb, z);
        else
            words[0] = quantize8<LG>(v[i][0], sb);
        if (e < slots) {
#pragma unroll
            for (int k = 0; k < V; ++k) packed[e * V + k] = words[k];
            if ((threadIdx.x & (LG - 1)) == 0) {
                scales[e / LG] = sb;
                if constexpr (ASYM) zeros[e / LG] = z;
            }
        }
    }
}

template <int LG, int CPT, bool ASYM, int EPL>
hipError_t launch_quantize_flat(const uint16_t* W, int64_t N, int64_t K, uint32_t* packed,
                                uint16_t* scales, int16_t* zeros, hipStream_t stream) {
    const int64_t slots = N * (K / EPL);
    const int64_t blocks = (slots + 256 * CPT - 1) / (256 * CPT);
    hipLaunchKernelGGL((quantize_flat_kernel<LG, CPT, ASYM, EPL>), dim3((unsigned)blocks),
                       dim3(256), 0, stream, reinterpret_cast<const uint4*>(W), slots, packed,
                       scales, zeros);
    return hipGetLastError();
}

hipError_t launch_quantize(const uint16_t* W, int64_t N, int64_t K, int64_t group,
                           uint32_t* packed, uint16_t* scales, hipStream_t stream, int num_cu,
                           const int* perm, int16_t* zeros) {
    if (N == 0 || K == 0) return hipSuccess;
    if (group == kPerChannel)
        return zeros != nullptr
                   ? launch_quantize_rows<true>(W, N, K, packed, scales, zeros, perm, stream)
                   : launch_quantize_rows<false>(W, N, K, packed, scales, nullptr, perm, stream);
    const int64_t groups = N * (K / group);
    if (groups == 0) return hipSuccess;
    // In their own column order: the flat grid (16 bytes a lane for
    // symmetric weights, 32 for asymmetric ones from group 64 up), up to 2^34
    // weights, where its work-items still fit the 32-bit grid size; larger
    // matrices take the persistent kernel below.
    const bool flat = perm == nullptr && N * K <= ((int64_t)1 << 34);
    if (zeros == nullptr && flat) {
        switch (group) {
            case 32: return launch_quantize_flat<4, 2, false, 8>(W, N, K, packed, scales, zeros,
                                                                 stream);
            case 64: return launch_quantize_flat<8, 2, false, 8>(W, N, K, packed, scales, zeros,
                                                                 stream);
            case 128: return launch_quantize_flat<16, 2, false, 8>(W, N, K, packed, scales, zeros,
                                                                   stream);
            case 256: return launch_quantize_flat<32, 2, false, 8>(W, N, K, packed, scales, zeros,
                                                                   stream);
            default: break;
        }
    }
    if (zeros != nullptr && flat) {
        switch (group) {
            case 32: return launch_quantize_flat<4, 1, true, 8>(W, N, K, packed, scales, zeros,
                                                                stream);
            case 64: return launch_quantize_flat<4, 1, true, 16>(W, N, K, packed, scales, zeros,
                                                                 stream);
            case 128: return launch_quantize_flat<8, 1, true, 16>(W, N, K, packed, scales, zeros,
                                                                  stream);
            case 256: return launch_quantize_flat<16, 1, true, 16>(W, N, K, packed, scales, zeros,
                                                                   stream);
            default: break;
        }
    }
    // Through act order (columns gathered through perm), or past 2^34
    // weights: the persistent kernel, 16 bytes a lane and U groups' loads a
    // step for every G.
    constexpr int U = kQuantizeGroupsPerStep;
    switch (group) {
        case 32:
            return launch_quantize_t<4, U>(W, groups, K, perm, packed, scales, zeros, stream, num_cu);
        case 64:
            return launch_quantize_t<8, U>(W, groups, K, perm, packed, scales, zeros, stream, num_cu);
        case 128:
            return launch_quantize_t<16, U>(W, groups, K, perm, packed, scales, zeros, stream,
                                            num_cu);
        case 256:
            return launch_quantize_t<32, U>(W, groups, K, perm, packed, scales, zeros, stream,
                                            num_cu);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace w4a16

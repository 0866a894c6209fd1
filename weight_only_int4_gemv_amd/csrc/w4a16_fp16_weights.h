// w4a16_fp16_weights.h — kernels whose MFMA B operand holds the dequantized
// weights fp16(s * q) ([QUANT] sub-section 3 dequantizer: s * q cast to fp16).
//
// With q in [-8, 7] and s = RNE_fp16(absmax / 7), s * q stays within the fp16
// range except in one case: a group whose absmax is 65504 (the largest
// finite fp16) has s = 9360 and s * 7 = 65520, a tie that rounds to
// infinity.  The exact weight is finite, so such groups' fp16 weights are
// clamped to +-65504 (error 16 in 65520, 2.4e-4 relative, inside the
// 1e-3 sum |x w| tolerance).  Scales below 9360 cannot reach the bound.
#pragma once

#include <type_traits>

#include "w4a16_device.h"

namespace w4a16 {

constexpr uint32_t kHugeScaleBits = 0x7092;   // fp16 9360

// True when a lane of the wave holds a group whose scale (fp16 bits s[tn])
// can push s * q past the fp16 range.  Wave-uniform: the caller picks one of
// two copies of its dequantize-and-multiply step, so the common copy has no
// branch between the dequantization and the MFMAs.
template <int TN>
__device__ __forceinline__ bool any_largest_scale(const uint32_t (&s)[TN]) {
    bool huge = false;
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) huge |= s[tn] >= kHugeScaleBits;
    return __any(huge);
}

// Clamp fp16 weights (bf: [tn][k-step]) to +-65504 (infinities included).
template <int TN>
__device__ __forceinline__ void clamp_fp16_weights(half8_t (&bf)[TN][4]) {
    const _Float16 m = (_Float16)65504.0f;
    const half8_t hi = {m, m, m, m, m, m, m, m};
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            bf[tn][kk] = __builtin_elementwise_max(__builtin_elementwise_min(bf[tn][kk], hi), -hi);
}

}  // namespace w4a16

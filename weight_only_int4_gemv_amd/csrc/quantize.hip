// quantize.hip — RTN symmetric INT4 quantizer, one fp16 scale per group of
// 128 along K, packed eight codes per uint32 ([QUANT] sub-section 2
// equations, sub-section 3 per-group listing; [INT4] INT4 paragraph).
//
// Work split: one 16-lane DPP row of a wave per (row, group).  Each lane loads
// 16 bytes (8 fp16), the row reduces the absolute maximum, and each lane
// writes the one packed word its 8 elements form; 16 lanes write the group's
// 64 contiguous bytes.  HBM traffic per element: 2 B in, 0.5 + 1/64 B out.
//
// Bit-exactness:
//   - |w| is compared as the integer w & 0x7FFF (order of finite fp16
//     magnitudes is the order of their bit patterns);
//   - s = fp16_rne(a / 7) with an IEEE fp32 division; double rounding
//     fp32 -> fp16 cannot change the result (24 >= 2*11 + 2);
//   - q = clamp(rint(w / s), -8, 7) with an IEEE fp32 division and rint
//     (half to even): for fp16 w and s a non-tie quotient is at least
//     2^-15 (relative) away from a tie, so the fp32 quotient rounds to the
//     same integer as the exact one.
#include "w4a16_device.h"
#include "w4a16_launch.h"

namespace w4a16 {

__global__ __launch_bounds__(256) void quantize_kernel(const uint4* __restrict__ W,
                                                       uint32_t* __restrict__ packed,
                                                       uint16_t* __restrict__ scales,
                                                       int64_t total_groups) {
    const int lane16 = threadIdx.x & 15;
    const int64_t stride = (int64_t)gridDim.x * (blockDim.x / 16);
    // The 16 lanes of a group always share g, so the row reductions below
    // only ever combine lanes that are active together.
    for (int64_t g = (int64_t)blockIdx.x * (blockDim.x / 16) + (threadIdx.x >> 4);
         g < total_groups; g += stride) {
        const uint4 v = W[g * 16 + lane16];  // 8 fp16 of this group
        uint32_t m = 0;
        m = max(m, v.x & 0x7FFFu);
        m = max(m, (v.x >> 16) & 0x7FFFu);
        m = max(m, v.y & 0x7FFFu);
        m = max(m, (v.y >> 16) & 0x7FFFu);
        m = max(m, v.z & 0x7FFFu);
        m = max(m, (v.z >> 16) & 0x7FFFu);
        m = max(m, v.w & 0x7FFFu);
        m = max(m, (v.w >> 16) & 0x7FFFu);
        // max over the 16 lanes of this group
        m = max(m, (uint32_t)__shfl_xor((int)m, 1, 16));
        m = max(m, (uint32_t)__shfl_xor((int)m, 2, 16));
        m = max(m, (uint32_t)__shfl_xor((int)m, 4, 16));
        m = max(m, (uint32_t)__shfl_xor((int)m, 8, 16));

        const float a = f16_bits_to_f32((uint16_t)m);
        const uint16_t s_bits = f32_to_f16_bits(a / 7.0f);  // 2^(4-1) - 1 = 7
        const float s = f16_bits_to_f32(s_bits);

        uint32_t word = 0x88888888u;  // every code 0 when s == 0
        if (s != 0.0f) {
            const uint32_t h[4] = {v.x, v.y, v.z, v.w};
            word = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint16_t b = (uint16_t)(h[i >> 1] >> (16 * (i & 1)));
                float r = rintf(f16_bits_to_f32(b) / s);
                r = fminf(fmaxf(r, -8.0f), 7.0f);
                word |= ((uint32_t)((int)r + 8) & 0xFu) << (4 * i);
            }
        }
        packed[g * 16 + lane16] = word;
        if (lane16 == 0) scales[g] = s_bits;
    }
}

hipError_t launch_quantize(const uint16_t* W, int64_t N, int64_t K, uint32_t* packed,
                           uint16_t* scales, hipStream_t stream) {
    const int64_t groups = N * (K / kGroup);
    if (groups == 0) return hipSuccess;
    const int threads = 256;                  // 16 groups per block
    int64_t blocks = (groups + 15) / 16;
    if (blocks > 65536) blocks = 65536;  // grid-stride beyond this
    hipLaunchKernelGGL(quantize_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream,
                       reinterpret_cast<const uint4*>(W), packed, scales, groups);
    return hipGetLastError();
}

}  // namespace w4a16

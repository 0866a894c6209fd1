// w4a16_launch.h — host-side launchers of the W4A16 kernels (private).
// Shapes are validated by the C ABI (api.hip) before any of these is called:
// 0 < M, N <= 2^24, 0 <= K < 2^31, K % 128 == 0, pointers aligned.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a16 {

hipError_t launch_quantize(const uint16_t* W, int64_t N, int64_t K, uint32_t* packed,
                           uint16_t* scales, hipStream_t stream);

// VALU dot-product path, any M (M > 8 runs in slices of 8 rows).
hipError_t launch_gemv_valu(const uint16_t* X, int64_t M, const uint32_t* packed,
                            const uint16_t* scales, int64_t N, int64_t K, uint16_t* Y,
                            hipStream_t stream, int num_cu);

// MFMA path, any M.
hipError_t launch_gemm_mfma(const uint16_t* X, int64_t M, const uint32_t* packed,
                            const uint16_t* scales, int64_t N, int64_t K, uint16_t* Y,
                            hipStream_t stream, int num_cu);

}  // namespace w4a16

// gather_x.hip — activations in the act-order column order ([QUANT] GPTQ
// section, act_order: the weight is stored with its columns in the order
// perm, and at inference the activations are permuted the same way).
//
// Xp[m, j] = X[m, perm[j]] (0 for an index outside [0, K)), so that a
// matrix-core GEMM over Xp and the stored weight computes
// Y[m,n] = sum_j X[m, perm[j]] * ŵ[n,j].  The prefill kernels stage X in
// 128-column steps; with a permuted order each step's columns lie anywhere in
// the row, so the gather is a pass of its own (2 M K bytes read, 2 M K
// written) rather than scattered 2-byte loads inside the GEMM's K loop.
//
// A block copies one row of X into LDS with 16-byte loads, then writes its
// share of the row's output columns, eight per thread per pass, reading
// perm with 16-byte loads and the values from LDS.  Rows longer than
// kGatherLdsMaxK are gathered from global memory (L2) directly.
#include "w4a16_device.h"
#include "w4a16_launch.h"

namespace w4a16 {

namespace {

constexpr int kGatherThreads = 256;
constexpr int64_t kGatherLdsMaxK = 32768;   // 64 KB of LDS per row

template <bool LDS>
__global__ __launch_bounds__(kGatherThreads) void gather_x_kernel(
    const uint16_t* __restrict__ X, const int* __restrict__ perm, uint16_t* __restrict__ Xp,
    int M, int K, int cols_per_block) {
    extern __shared__ uint4 row_lds[];
    const int j0 = blockIdx.x * cols_per_block;
    const int j1 = min(K, j0 + cols_per_block);
    for (int m = blockIdx.y; m < M; m += gridDim.y) {
        const uint16_t* xrow = X + (size_t)m * K;
        if constexpr (LDS) {
            __syncthreads();    // the previous row's reads are done
            const uint4* src = reinterpret_cast<const uint4*>(xrow);
            for (int v = threadIdx.x; v < K / 8; v += kGatherThreads) row_lds[v] = src[v];
            __syncthreads();
        }
        const uint16_t* from = LDS ? reinterpret_cast<const uint16_t*>(row_lds) : xrow;
        for (int j = j0 + (int)threadIdx.x * 8; j < j1; j += kGatherThreads * 8) {
            const int4 p0 = reinterpret_cast<const int4*>(perm + j)[0];
            const int4 p1 = reinterpret_cast<const int4*>(perm + j)[1];
            const int p[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
            uint32_t h[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) h[i] = (uint32_t)p[i] < (uint32_t)K ? from[p[i]] : 0u;
            reinterpret_cast<uint4*>(Xp + (size_t)m * K + j)[0] =
                make_uint4(h[0] | h[1] << 16, h[2] | h[3] << 16, h[4] | h[5] << 16,
                           h[6] | h[7] << 16);
        }
    }
}

}  // namespace

hipError_t launch_gather_x(const uint16_t* X, int64_t M, int64_t K, const int* perm,
                           uint16_t* Xp, hipStream_t stream, int num_cu) {
    if (M <= 0 || K <= 0) return hipSuccess;
    // Column blocks per row: one when the rows alone give every compute unit
    // two blocks, else enough to (at >= 2048 columns a block).
    int64_t chunks = 1;
    if (M < 2 * (int64_t)num_cu) {
        chunks = (2 * num_cu + M - 1) / M;
        chunks = chunks < K / 2048 ? chunks : (K / 2048 > 0 ? K / 2048 : 1);
    }
    int64_t cols = (K + chunks - 1) / chunks;
    cols = (cols + 7) / 8 * 8;
    chunks = (K + cols - 1) / cols;
    const dim3 grid((unsigned)chunks, (unsigned)(M < 65535 ? M : 65535));
    if (K <= kGatherLdsMaxK) {
        hipLaunchKernelGGL(gather_x_kernel<true>, grid, dim3(kGatherThreads), (size_t)K * 2,
                           stream, X, perm, Xp, (int)M, (int)K, (int)cols);
    } else {
        hipLaunchKernelGGL(gather_x_kernel<false>, grid, dim3(kGatherThreads), 0, stream, X,
                           perm, Xp, (int)M, (int)K, (int)cols);
    }
    return hipGetLastError();
}

}  // namespace w4a16

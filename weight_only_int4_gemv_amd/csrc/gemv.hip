// gemv.hip — decode GEMV (M = 1) and small-M VALU GEMV for W4A16.
//
// y[m,n] = sum_g s[n,g] * sum_{k in g} q[n,k] x[m,k], fp32 accumulation,
// fp16 output ([BENCH] §二: decode streams every weight once and is
// memory-bound; §五: dequantize on the fly in registers, never in memory).
//
// Design for gfx950 (HBM3E-bound streaming, VALU kept below its limit):
//   - Activations are staged once per block into LDS, in the paired order of
//     pair_block().  Slices of K are staged in turn when M * K does not fit
//     the LDS budget.
//   - Each wave owns R consecutive rows.  Its 64 lanes walk K in 16-byte
//     chunks (32 codes), lane l taking chunks l, l+64, ...: every load
//     instruction of the wave reads R fully used, contiguous 1 KiB spans.
//     U chunk steps of all R rows are loaded before any is consumed.
//   - A word of 8 codes costs one shift, four v_and_or_b32 and four packed
//     fp16 add/fma to form the codes exactly in fp16 (codes_word), then four
//     v_dot2_f32_f16 per activation row; per chunk one fma applies the group
//     scale to the chunk's partial sum.
//   - Partial sums are reduced across the wave with butterfly shuffles and
//     the result is rounded once to fp16.
// Precision: every product q*x is exact in fp32, so accumulation error is
// relative to sum |q x| (within the 1e-3 sum |x w| allowance for every K);
// a one-hot x reproduces fp16(s*q) exactly.
#include "w4a16_device.h"
#include "w4a16_launch.h"

namespace w4a16 {

namespace {

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

// Stage activation rows [0, M) x elements [k0, k0 + ks) into LDS:
//   xs[m * (ks/8) + b] = paired 8-element block b of the slice.
__device__ __forceinline__ void stage_activations(const uint16_t* __restrict__ X, int M, int K,
                                                  int k0, int ks, uint4* xs) {
    const int nblk = ks >> 3;
    for (int i = threadIdx.x; i < M * nblk; i += blockDim.x) {
        const int m = i / nblk;
        const int b = i - m * nblk;
        const uint4 v = reinterpret_cast<const uint4*>(X + (size_t)m * K + k0)[b];
        xs[m * nblk + b] = pair_block(v.x, v.y, v.z, v.w);
    }
}

}  // namespace

// MMAX: activation rows handled (M <= MMAX at run time).  R: weight rows per
// wave.  U: chunk steps loaded ahead.  WAVES: waves per block.
template <int MMAX, int R, int U, int WAVES>
__global__ __launch_bounds__(WAVES * kWave) void gemv_kernel(
    const uint16_t* __restrict__ X, int M, const uint4* __restrict__ packed,
    const uint16_t* __restrict__ scales, uint16_t* __restrict__ Y, int N, int K, int kslice) {
    extern __shared__ uint4 lds[];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int nchunks = K >> 5;   // 16-byte chunks per weight row
    const int ngroups = K >> 7;   // scales per weight row
    const int row0 = (blockIdx.x * WAVES + wave) * R;

    int rows[R];
#pragma unroll
    for (int r = 0; r < R; ++r) rows[r] = min(row0 + r, N - 1);  // tail rows re-read row N-1

    float acc[MMAX][R];
#pragma unroll
    for (int m = 0; m < MMAX; ++m)
#pragma unroll
        for (int r = 0; r < R; ++r) acc[m][r] = 0.0f;

    for (int k0 = 0; k0 < K; k0 += kslice) {
        const int ks = min(kslice, K - k0);
        const int c0 = k0 >> 5;          // first chunk of the slice
        const int nch = ks >> 5;
        uint4* xs = lds;
        if (k0 > 0) __syncthreads();     // previous slice fully consumed
        stage_activations(X, M, K, k0, ks, xs);
        __syncthreads();

        for (int cbase = lane; cbase < nch; cbase += U * kWave) {
            // All U*R loads are issued before the first is used; a step past
            // the slice end re-reads the last chunk (in bounds) and is skipped.
            uint4 w[U][R];
            uint16_t sb[U][R];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int cc = c0 + min(cbase + u * kWave, nch - 1);
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    w[u][r] = packed[(size_t)rows[r] * nchunks + cc];
                    sb[u][r] = scales[(size_t)rows[r] * ngroups + (cc >> 2)];
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = cbase + u * kWave;
                if (c >= nch) break;
#pragma unroll
                for (int m = 0; m < MMAX; ++m) {
                    if (m >= M) break;
                    const uint4* xp = xs + m * (ks >> 3) + c * 4;
                    const uint4 x0 = xp[0], x1 = xp[1], x2 = xp[2], x3 = xp[3];
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        float part = dot_word(w[u][r].x, x0, 0.0f);
                        part = dot_word(w[u][r].y, x1, part);
                        part = dot_word(w[u][r].z, x2, part);
                        part = dot_word(w[u][r].w, x3, part);
                        acc[m][r] = fmaf(f16_bits_to_f32(sb[u][r]), part, acc[m][r]);
                    }
                }
            }
        }
    }

#pragma unroll
    for (int m = 0; m < MMAX; ++m) {
        if (m >= M) break;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float v = wave_sum(acc[m][r]);
            if (lane == 0 && row0 + r < N) Y[(size_t)m * N + row0 + r] = f32_to_f16_bits(v);
        }
    }
}

namespace {

constexpr int kLdsBudget = 64 * 1024;

template <int MMAX, int R, int U, int WAVES>
hipError_t launch_gemv_t(const uint16_t* X, int64_t M, const uint32_t* packed,
                         const uint16_t* scales, int64_t N, int64_t K, uint16_t* Y,
                         hipStream_t stream) {
    // LDS: 2 bytes per activation element.
    int64_t kslice = (int64_t)(kLdsBudget / (MMAX * 2)) / kGroup * kGroup;
    if (kslice > K) kslice = K;
    if (kslice < kGroup) kslice = kGroup;
    const size_t lds = (size_t)MMAX * (kslice / 8) * sizeof(uint4);
    const int64_t rows_per_block = (int64_t)R * WAVES;
    const int64_t blocks = (N + rows_per_block - 1) / rows_per_block;
    hipLaunchKernelGGL((gemv_kernel<MMAX, R, U, WAVES>), dim3((unsigned)blocks),
                       dim3(WAVES * kWave), lds, stream, X, (int)M,
                       reinterpret_cast<const uint4*>(packed), scales, Y, (int)N, (int)K,
                       (int)kslice);
    return hipGetLastError();
}

// Rows per wave: as many as keep at least two blocks per compute unit.
template <int MMAX>
hipError_t launch_gemv_m(const uint16_t* X, int64_t M, const uint32_t* packed,
                         const uint16_t* scales, int64_t N, int64_t K, uint16_t* Y,
                         hipStream_t stream, int num_cu) {
    constexpr int WAVES = 4;
    if (N >= (int64_t)4 * WAVES * num_cu)
        return launch_gemv_t<MMAX, 4, 2, WAVES>(X, M, packed, scales, N, K, Y, stream);
    if (N >= (int64_t)2 * WAVES * num_cu)
        return launch_gemv_t<MMAX, 2, 2, WAVES>(X, M, packed, scales, N, K, Y, stream);
    return launch_gemv_t<MMAX, 1, 4, WAVES>(X, M, packed, scales, N, K, Y, stream);
}

}  // namespace

hipError_t launch_gemv_valu(const uint16_t* X, int64_t M, const uint32_t* packed,
                            const uint16_t* scales, int64_t N, int64_t K, uint16_t* Y,
                            hipStream_t stream, int num_cu) {
    if (M == 1) return launch_gemv_m<1>(X, M, packed, scales, N, K, Y, stream, num_cu);
    if (M == 2) return launch_gemv_m<2>(X, M, packed, scales, N, K, Y, stream, num_cu);
    if (M <= 4) return launch_gemv_m<4>(X, M, packed, scales, N, K, Y, stream, num_cu);
    // M > 8 is split into slices of at most 8 activation rows.
    for (int64_t m0 = 0; m0 < M; m0 += 8) {
        const int64_t mm = (M - m0 < 8) ? (M - m0) : 8;
        hipError_t e = launch_gemv_m<8>(X + m0 * K, mm, packed, scales, N, K, Y + m0 * N,
                                        stream, num_cu);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace w4a16

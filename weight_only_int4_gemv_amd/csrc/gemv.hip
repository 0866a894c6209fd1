// gemv.hip — decode GEMV (M = 1) and small-M VALU GEMV for W4A16.
//
// y[m,n] = sum_g s[n,g] * sum_{k in g} q[n,k] x[m,k], fp32 accumulation,
// fp16 output ([BENCH] §二: decode streams every weight once and is
// memory-bound; §五: dequantize on the fly in registers, never in memory).
//
// Design for gfx950 (HBM3E-bound streaming, VALU kept well below its limit):
//   - Activations are staged once per block into LDS, in the paired order of
//     pair_block(), with two per-chunk offsets that remove the +8 of the
//     codes (see dot_word_nibbles).  Slices of K are staged in turn when
//     M * K does not fit the LDS budget.
//   - Each wave owns R consecutive rows.  Its 64 lanes walk K in 16-byte
//     chunks (32 codes), lane l taking chunks l, l+64, ...: every load
//     instruction of the wave reads R fully used, contiguous 1 KiB spans.
//     U chunk steps of all R rows are loaded before any is consumed.
//   - A chunk costs 4 shifts, 16 ANDs and 16 v_dot2_f32_f16 per row and per
//     activation row: the nibble read as an fp16 subnormal is n * 2^-24 (or
//     n * 2^-20 for the nibbles at bits 4-7), so no conversion instruction
//     is needed.  Per chunk, one fma folds the two accumulators and one fma
//     applies the group scale.
//   - Partial sums are reduced across the wave with butterfly shuffles; the
//     result (scaled back by 2^24) is rounded once to fp16.
// Precision: the offsets are removed per 32-element chunk, so accumulated
// magnitudes stay those of sum |q x| (codes <= 15 in magnitude, never the
// 1032 of magic-number unpacking); a one-hot x is reproduced exactly.
#include "w4a16_device.h"
#include "w4a16_launch.h"

namespace w4a16 {

namespace {

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

// Stage activation rows [0, M) x elements [k0, k0 + ks) into LDS.
//   xs[m * (ks/8) + b]   paired 8-element block b of the slice
//   xb[m * (ks/32) + c]  (-8 * 2^-24 * lo-sum, -8 * 2^-20 * hi-sum) of chunk c
__device__ __forceinline__ void stage_activations(const uint16_t* __restrict__ X, int M, int K,
                                                  int k0, int ks, uint4* xs, float2* xb) {
    const int nch = ks >> 5;
    for (int i = threadIdx.x; i < M * nch; i += blockDim.x) {
        const int m = i / nch;
        const int c = i - m * nch;
        const uint4* src = reinterpret_cast<const uint4*>(X + (size_t)m * K + k0) + c * 4;
        uint4 p[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const uint4 v = src[b];
            p[b] = pair_block(v.x, v.y, v.z, v.w);
            xs[m * (ks >> 3) + c * 4 + b] = p[b];
        }
        const float2 sums = chunk_sums(p);
        xb[m * nch + c] = make_float2(-8.0f * 0x1p-24f * sums.x, -8.0f * 0x1p-20f * sums.y);
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
        float2* xb = reinterpret_cast<float2*>(lds + MMAX * (kslice >> 3));
        if (k0 > 0) __syncthreads();     // previous slice fully consumed
        stage_activations(X, M, K, k0, ks, xs, xb);
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
                    const float2 bias = xb[m * nch + c];
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        float lo = bias.x, hi = bias.y;
                        dot_word_nibbles(w[u][r].x, x0, lo, hi);
                        dot_word_nibbles(w[u][r].y, x1, lo, hi);
                        dot_word_nibbles(w[u][r].z, x2, lo, hi);
                        dot_word_nibbles(w[u][r].w, x3, lo, hi);
                        // lo + 16 hi = 2^-24 * sum_k q_k x_k over the chunk
                        acc[m][r] = fmaf(f16_bits_to_f32(sb[u][r]), fmaf(hi, 16.0f, lo), acc[m][r]);
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
            if (lane == 0 && row0 + r < N) Y[(size_t)m * N + row0 + r] = f32_to_f16_bits(v * 0x1p24f);
        }
    }
}

namespace {

constexpr int kLdsBudget = 64 * 1024;

template <int MMAX, int R, int U, int WAVES>
hipError_t launch_gemv_t(const uint16_t* X, int64_t M, const uint32_t* packed,
                         const uint16_t* scales, int64_t N, int64_t K, uint16_t* Y,
                         hipStream_t stream) {
    // LDS per activation element: 2 B of x plus 8 B of offsets per 32.
    int64_t kslice = (int64_t)(kLdsBudget / (MMAX * 2.25)) / kGroup * kGroup;
    if (kslice > K) kslice = K;
    if (kslice < kGroup) kslice = kGroup;
    const size_t lds = (size_t)MMAX * (kslice / 8) * sizeof(uint4) +
                       (size_t)MMAX * (kslice / 32) * sizeof(float2);
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

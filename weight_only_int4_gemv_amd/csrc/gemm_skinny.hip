// gemm_skinny.hip — W4A16 GEMM for few rows of X (batched decode, M = 3..64):
// Y[m,n] = sum_k X[m,k] * fp16(s[n,k/128] * q[n,k]) on the matrix cores,
// streaming the weights like the decode GEMV ([BENCH] §二: decode reads every
// weight once and is bound by memory; batching several tokens reuses each
// weight for all of them).
//
// Layout of work: a block owns 16*TN weight rows (MFMA N tiles) and 16*TM
// rows of X; its WK waves split the K groups into contiguous ranges; the
// partial tiles are summed through LDS in a fixed order (deterministic).
// No LDS staging and no barriers inside the K loop:
//   - B: lane (n = l%16, j = l/16) loads words 4j..4j+3 of its row's group
//     (one 16-byte non-temporal buffer load per N tile) and dequantizes them
//     to fp16(s*q) in the paired order of dequant_word — word 4j+kk is its
//     B operand for k-step kk of v_mfma_f32_16x16x32_f16;
//   - A: lane (m = l%16, j) loads the 32 activations of row m that the same
//     k-steps cover (four 16-byte buffer loads, L2-resident) and pairs them
//     (pair_block) to match;
//   - the (group) iterations run through a ring of P+1 register slots,
//     loads for group t+P issued before group t is multiplied; loads past a
//     wave's range use an empty buffer resource, and rows past M or N read 0;
//   - a wave whose group holds absmax 65504 (s = 9360: 7 s rounds to
//     infinity in fp16) runs a copy of the step that clamps its fp16
//     weights to +-65504 (error 16 in 65520).
#include "w4a16_device.h"
#include "w4a16_launch.h"
#include "w4a16_fp16_weights.h"

namespace w4a16 {

template <int TM, int TN, int WK, int P>
__global__ __launch_bounds__(WK * kWave) void gemm_skinny_kernel(
    const uint16_t* __restrict__ X, int M, const uint32_t* __restrict__ packed,
    const uint16_t* __restrict__ scales, uint16_t* __restrict__ Y, int N, int K) {
    constexpr int Q = P + 1;
    extern __shared__ float4_t red[];                  // (WK-1) x TM*TN x 64 partial tiles
    const int lane = threadIdx.x & (kWave - 1);
    const int wk = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int l16 = lane & 15;
    const int j = lane >> 4;
    const int n0 = blockIdx.x * 16 * TN;
    const int m0 = blockIdx.y * 16 * TM;
    const int ngroups = K >> 7;
    const int g_begin = (int)((int64_t)ngroups * wk / WK);
    const int g_end = (int)((int64_t)ngroups * (wk + 1) / WK);
    const int Tw = g_end - g_begin;                     // this wave's groups
    const uint32_t wrow = (uint32_t)K / 2, srow = (uint32_t)K / 64, xrow = (uint32_t)K * 2;
    const CodeConsts kc = code_consts();

    const __amdgpu_buffer_rsrc_t wr_live = buffer_rsrc(
        reinterpret_cast<const char*>(packed) + (size_t)n0 * wrow, (uint64_t)(N - n0) * wrow);
    const __amdgpu_buffer_rsrc_t sr_live = buffer_rsrc(
        reinterpret_cast<const char*>(scales) + (size_t)n0 * srow, (uint64_t)(N - n0) * srow);
    const __amdgpu_buffer_rsrc_t xr_live = buffer_rsrc(
        reinterpret_cast<const char*>(X) + (size_t)m0 * xrow, (uint64_t)(M - m0) * xrow);
    const __amdgpu_buffer_rsrc_t empty = buffer_rsrc(packed, 0);

    typedef unsigned v4u __attribute__((ext_vector_type(4)));
    // scales in 32-bit slots: 16-bit slots would be packed in pairs, and
    // packing waits for both loads
    struct Slot {
        v4u b[TN];
        uint32_t s[TN];
        v4u a[TM][4];
    };
    // Blocks start their K ranges at different groups so that they do not
    // all read the same activations at the same time; loads are issued in
    // order t = 0, 1, ... and the cursor wraps inside [g_begin, g_end).
    int gl = Tw > 0 ? g_begin + (int)(blockIdx.x % (unsigned)Tw) : g_begin;
    auto load = [&](int t, Slot& sl) {
        const bool live = t < Tw;
        const __amdgpu_buffer_rsrc_t wr = live ? wr_live : empty;
        const __amdgpu_buffer_rsrc_t sr = live ? sr_live : empty;
        const __amdgpu_buffer_rsrc_t xr = live ? xr_live : empty;
        const int g = gl;
        if (++gl == g_end) gl = g_begin;
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
            const int row = tn * 16 + l16;
            sl.b[tn] = __builtin_amdgcn_raw_buffer_load_b128(wr, row * wrow + g * 64 + j * 16, 0,
                                                             kStreamLoad);
            sl.s[tn] = __builtin_amdgcn_raw_buffer_load_b16(sr, row * srow + g * 2, 0, kStreamLoad);
        }
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) {
            const int voff = (tm * 16 + l16) * xrow + g * 256 + j * 64;
#pragma unroll
            for (int u = 0; u < 4; ++u)
                sl.a[tm][u] = __builtin_amdgcn_raw_buffer_load_b128(xr, voff + u * 16, 0, 0);
        }
    };

    float4_t acc[TM][TN];
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) acc[tm][tn] = (float4_t){0.f, 0.f, 0.f, 0.f};

    Slot ring[Q];
#pragma unroll
    for (int i = 0; i < P; ++i) load(i, ring[i]);

    for (int t0 = 0; t0 < Tw; t0 += Q) {
#pragma unroll
        for (int i = 0; i < Q; ++i) {
            load(t0 + i + P, ring[(i + P) % Q]);
            if (t0 + i >= Tw) continue;                  // wave-uniform
            const Slot& sl = ring[i];
            auto mma = [&](auto clamp) __attribute__((always_inline)) {
                half8_t bf[TN][4];
#pragma unroll
                for (int tn = 0; tn < TN; ++tn) {
                    const _Float16 sh = __builtin_bit_cast(_Float16, (uint16_t)sl.s[tn]);
                    const half2_t s2 = {sh, sh};
                    const uint32_t words[4] = {sl.b[tn].x, sl.b[tn].y, sl.b[tn].z, sl.b[tn].w};
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk) {
                        half2_t h[4];
                        dequant_word(words[kk], s2, h, kc);
                        bf[tn][kk] = (half8_t){h[0].x, h[0].y, h[1].x, h[1].y,
                                               h[2].x, h[2].y, h[3].x, h[3].y};
                    }
                }
                if constexpr (decltype(clamp)::value) clamp_fp16_weights(bf);
#pragma unroll
                for (int tm = 0; tm < TM; ++tm) {
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk) {
                        const v4u v = sl.a[tm][kk];
                        const half8_t af =
                            __builtin_bit_cast(half8_t, pair_block(v.x, v.y, v.z, v.w));
#pragma unroll
                        for (int tn = 0; tn < TN; ++tn)
                            acc[tm][tn] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                                af, bf[tn][kk], acc[tm][tn], 0, 0, 0);
                    }
                }
            };
            if (any_largest_scale(sl.s))
                mma(std::true_type{});
            else
                mma(std::false_type{});
        }
    }

    // Sum the WK partial tiles in a fixed order, then store.
    if constexpr (WK > 1) {
        if (wk > 0) {
#pragma unroll
            for (int tm = 0; tm < TM; ++tm)
#pragma unroll
                for (int tn = 0; tn < TN; ++tn)
                    red[((wk - 1) * TM * TN + tm * TN + tn) * kWave + lane] = acc[tm][tn];
        }
        __syncthreads();
        if (wk > 0) return;
#pragma unroll
        for (int w = 1; w < WK; ++w)
#pragma unroll
            for (int tm = 0; tm < TM; ++tm)
#pragma unroll
                for (int tn = 0; tn < TN; ++tn)
                    acc[tm][tn] += red[((w - 1) * TM * TN + tm * TN + tn) * kWave + lane];
    }
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
            const int n = n0 + tn * 16 + l16;
            if (n >= N) continue;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + tm * 16 + 4 * j + r;
                if (m < M) Y[(size_t)m * N + n] = f32_to_f16_bits(acc[tm][tn][r]);
            }
        }
    }
}

template <int TM, int TN, int WK, int P>
hipError_t launch_skinny_t(const uint16_t* X, int64_t M, const uint32_t* packed,
                           const uint16_t* scales, int64_t N, int64_t K, uint16_t* Y,
                           hipStream_t stream) {
    const size_t lds = (size_t)(WK > 1 ? WK - 1 : 1) * TM * TN * kWave * sizeof(float4_t);
    const dim3 grid((unsigned)((N + 16 * TN - 1) / (16 * TN)),
                    (unsigned)((M + 16 * TM - 1) / (16 * TM)));
    hipLaunchKernelGGL((gemm_skinny_kernel<TM, TN, WK, P>), grid, dim3(WK * kWave), lds, stream,
                       X, (int)M, packed, scales, Y, (int)N, (int)K);
    return hipGetLastError();
}

hipError_t launch_gemm_skinny(const uint16_t* X, int64_t M, const uint32_t* packed,
                              const uint16_t* scales, int64_t N, int64_t K, uint16_t* Y,
                              hipStream_t stream, int num_cu) {
    (void)num_cu;
    // Measured on gfx950 (down projection 14336 x 4096): one 16-row tile per
    // wave, four waves over K, three groups in flight up to M = 16; two
    // M tiles per wave up to 32; two M and two N tiles beyond.
    if (M <= 16) return launch_skinny_t<1, 1, 4, 3>(X, M, packed, scales, N, K, Y, stream);
    if (M <= 32) return launch_skinny_t<2, 1, 4, 2>(X, M, packed, scales, N, K, Y, stream);
    return launch_skinny_t<2, 2, 4, 1>(X, M, packed, scales, N, K, Y, stream);
}

}  // namespace w4a16

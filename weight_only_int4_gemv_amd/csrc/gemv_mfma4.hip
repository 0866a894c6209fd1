// gemv_mfma4.hip — W4A16 GEMV for few rows of X (decode and batched decode,
// M = 1..16) that streams the weights like the VALU GEMV but multiplies on
// the matrix cores ([BENCH] §二: decode is bound by reading every weight
// once; [QUANT] dequantization s * q per group of 128).
//
// v_mfma_f32_4x4x4_16b_f16 computes 16 independent 4x4x4 products.  Lane
// l = 4b + c belongs to block b; it supplies row c of block b's A (4 k
// values) and column c of block b's B (the same 4 k), and receives column c
// of block b's D (rows in its 4 result registers).
//
// Mapping: a wave owns 4 weight rows (n0 + c for lane 4b + c) and walks K in
// steps of 512 * U.  Lane 4b + c loads 16 bytes of row n0 + c per step and
// load (32 codes: k0 + 32b .. k0 + 32b + 31), so one load instruction reads
// 256 contiguous bytes of each of the 4 rows.  The 32 codes (exact fp16
// integers in the paired order of codes_word) are the B operand of eight
// MFMA steps; for every step all four lanes of block b use the same 4 k, so
// block b's A is x at those k for up to 4 tokens (token c in lane 4b + c),
// read from LDS where x is staged in the same paired order.  A group of 128
// never straddles a lane's 32 codes, so the eight steps' D is one group's
// partial dot product per (token, row): it is multiplied by that group's
// scale once (fp32 FMA) — products and sums inside the MFMA are exact fp16
// products accumulated in fp32, as in the VALU GEMV.  At the end of a row
// the 16 blocks' partial sums are added across lanes 4b + c (fixed order)
// and lanes 0..3 store the row's outputs.  Up to MT sets of 4 tokens share
// every weight load.
//
// Steps run through a ring of P + 1 register slots as in the VALU GEMV:
// the loads of step t + P are issued before step t is multiplied; loads past
// the wave's work use an empty buffer resource, rows past N and codes past K
// read as 0 and are given scale 0.
//
// Few row groups for the compute units (short N, long K: the down
// projection has N / 4 = 1024 row groups, one wave per SIMD): KS > 1 waves
// share each row group, wave part p taking the steps p, p + KS, ... (the
// same number for every part; steps past K load nothing useful and get
// scale 0).  A block then works through batches of WAVES / KS row groups,
// the same number of batches for every wave of the block, and at the end of
// each batch parts 1 .. KS-1 leave their partial sums in LDS, part 0 adds
// them in that order and stores: two barriers per batch, reached by every
// wave.
#include "w4a16_device.h"
#include "w4a16_launch.h"

namespace w4a16 {

namespace {
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ half4_t as_h4(uint32_t lo, uint32_t hi) {
    typedef uint32_t u2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(half4_t, (u2){lo, hi});
}

// Sum over the 16 lanes 4b + c (b = 0..15) of every c; the sums end in
// lanes 0..3.  Rotations by 4 and 8 inside each row of 16 lanes, then the
// four rows are added with cross-row swizzles.
__device__ __forceinline__ float block_sum(float v) {
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, false));  // row_ror:4
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false));  // row_ror:8
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    return v;
}
}  // namespace

template <int MT, int U, int P, int WAVES, int KS>
__global__ __launch_bounds__(WAVES * kWave) void gemv_mfma4_kernel(
    const uint16_t* __restrict__ X, int M, const uint32_t* __restrict__ packed,
    const uint16_t* __restrict__ scales, uint16_t* __restrict__ Y, int N, int K) {
    extern __shared__ uint4 lds[];                    // [M][K/8 + 1] paired x, then
                                                      // (KS > 1) partial sums
    static_assert(WAVES % KS == 0, "waves per row group must divide the block");
    constexpr int RGB = WAVES / KS;                   // row groups per block and batch
    constexpr int Q = P + 1;
    constexpr int kRows = 4;
    constexpr int kStepK = 512 * U;                   // k per step
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int b = lane >> 2;
    const int c = lane & 3;
    const int part = wave % KS;                       // this wave's share of the K steps
    const int nsteps = (K + kStepK - 1) / kStepK;
    const int spw = (nsteps + KS - 1) / KS;           // steps per wave and row group
    const int total_rg = (N + kRows - 1) / kRows;
    const int stride_rg = gridDim.x * RGB;
    const int first_rg = blockIdx.x * RGB + wave / KS;
    // KS == 1: each wave's own row groups.  KS > 1: the block's batches,
    // counted from its first row group, so every wave runs the same loop.
    const int sched_rg = KS == 1 ? first_rg : (int)blockIdx.x * RGB;
    const int my_rg = sched_rg < total_rg ? (total_rg - 1 - sched_rg) / stride_rg + 1 : 0;
    const int T = my_rg * spw;
    const int xblk = K >> 3;                          // 8-element blocks per x row
    const int xstride = xblk + 1;                     // 16-byte pad: rows start 4 banks apart
    const uint32_t wrow = (uint32_t)K / 2, srow = (uint32_t)K / 64;
    const CodeConsts kc = code_consts();

    // stage X into LDS in the paired order
    {
        const int total = M * xblk;
        for (int i0 = threadIdx.x; i0 < total; i0 += 4 * WAVES * kWave) {
            uint4 v[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int i = min(i0 + j * WAVES * kWave, total - 1);
                v[j] = reinterpret_cast<const uint4*>(X)[i];
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int i = i0 + j * WAVES * kWave;
                if (i < total) lds[i + i / xblk] = pair_block(v[j].x, v[j].y, v[j].z, v[j].w);
            }
        }
    }

    // load cursor (wave-uniform): iteration tl -> (row group lrg, step ls)
    int tl = 0, lrg = first_rg, ls = 0;
    __amdgpu_buffer_rsrc_t wr = buffer_rsrc(packed, 0), sr = buffer_rsrc(scales, 0);
    typedef unsigned v4u __attribute__((ext_vector_type(4)));
    // scales in 32-bit slots: 16-bit slots would be packed in pairs, and
    // packing waits for both loads
    auto load = [&](v4u (&wd)[U], uint32_t (&sd)[U]) {
        if (ls == 0) {
            const int64_t row0 = (int64_t)lrg * kRows;
            const bool live = tl < T && row0 < N;
            const int64_t rows_left = live ? (int64_t)N - row0 : 0;
            wr = buffer_rsrc(reinterpret_cast<const char*>(packed) + (live ? row0 * wrow : 0),
                             (uint64_t)rows_left * wrow);
            sr = buffer_rsrc(reinterpret_cast<const char*>(scales) + (live ? row0 * srow : 0),
                             (uint64_t)rows_left * srow);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int k = (part + KS * ls) * kStepK + u * 512 + b * 32;   // this lane's first k
            const uint32_t kk = (uint32_t)min(k, K);               // past K: reads as 0
            wd[u] = __builtin_amdgcn_raw_buffer_load_b128(wr, c * wrow + kk / 2, 0, kStreamLoad);
            sd[u] = __builtin_amdgcn_raw_buffer_load_b16(sr, c * srow + (kk >> 7) * 2, 0,
                                                         kStreamLoad);
        }
        ++tl;
        if (++ls == spw) {
            ls = 0;
            lrg += stride_rg;
        }
    };

    v4u wq[Q][U];
    uint32_t sq[Q][U];
#pragma unroll
    for (int i = 0; i < P; ++i) load(wq[i], sq[i]);
    __syncthreads();

    int crg = first_rg, cs = 0;
    float4_t acc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[t] = (float4_t){0.f, 0.f, 0.f, 0.f};

    for (int t0 = 0; t0 < T; t0 += Q) {
#pragma unroll
        for (int i = 0; i < Q; ++i) {
            load(wq[(i + P) % Q], sq[(i + P) % Q]);
            if (t0 + i < T) {                                      // wave-uniform
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int k = (part + KS * cs) * kStepK + u * 512 + b * 32;
                    const bool valid = k < K;
                    const int blk = min(k, K - 32) >> 3;           // x of a valid chunk
                    const uint32_t words[4] = {wq[i][u].x, wq[i][u].y, wq[i][u].z, wq[i][u].w};
                    float4_t d[MT];
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        half2_t q[4];
                        codes_word(words[w], kc, q);
                        const half4_t b0 = as_h4(as_u32(q[0]), as_u32(q[1]));
                        const half4_t b1 = as_h4(as_u32(q[2]), as_u32(q[3]));
#pragma unroll
                        for (int t = 0; t < MT; ++t) {
                            const int m = t * 4 + c;
                            const uint4 xv = m < M ? lds[m * xstride + blk + w] : make_uint4(0, 0, 0, 0);
                            const half4_t a0 = as_h4(xv.x, xv.y);
                            const half4_t a1 = as_h4(xv.z, xv.w);
                            if (w == 0)
                                d[t] = __builtin_amdgcn_mfma_f32_4x4x4f16(
                                    a0, b0, (float4_t){0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                            else
                                d[t] = __builtin_amdgcn_mfma_f32_4x4x4f16(a0, b0, d[t], 0, 0, 0);
                            d[t] = __builtin_amdgcn_mfma_f32_4x4x4f16(a1, b1, d[t], 0, 0, 0);
                        }
                    }
                    const float sc = valid ? f16_bits_to_f32((uint16_t)sq[i][u]) : 0.0f;
#pragma unroll
                    for (int t = 0; t < MT; ++t) {
                        acc[t][0] = fmaf(sc, d[t][0], acc[t][0]);
                        acc[t][1] = fmaf(sc, d[t][1], acc[t][1]);
                        acc[t][2] = fmaf(sc, d[t][2], acc[t][2]);
                        acc[t][3] = fmaf(sc, d[t][3], acc[t][3]);
                    }
                }
            }
            if (++cs == spw) {
                cs = 0;
                if (t0 + i < T) {                                  // block-uniform for KS > 1
                    if constexpr (KS > 1) {
                        // parts 1 .. KS-1 publish, part 0 adds them in order
                        float4_t* red = reinterpret_cast<float4_t*>(lds + M * xstride) +
                                        (size_t)(wave / KS) * (KS - 1) * MT * kWave;
                        if (part > 0) {
#pragma unroll
                            for (int t = 0; t < MT; ++t)
                                red[((part - 1) * MT + t) * kWave + lane] = acc[t];
                        }
                        __syncthreads();
                        if (part == 0) {
                            for (int p = 1; p < KS; ++p)
#pragma unroll
                                for (int t = 0; t < MT; ++t)
                                    acc[t] += red[((p - 1) * MT + t) * kWave + lane];
                        }
                    }
                    if (part == 0) {
                        // row group complete: add the 16 blocks, lanes 0..3 store
                        const int row = crg * kRows + c;
#pragma unroll
                        for (int t = 0; t < MT; ++t) {
#pragma unroll
                            for (int r = 0; r < 4; ++r) {
                                const float v = block_sum(acc[t][r]);
                                const int m = t * 4 + r;
                                if (lane < 4 && m < M && row < N)
                                    Y[(size_t)m * N + row] = f32_to_f16_bits(v);
                            }
                        }
                    }
#pragma unroll
                    for (int t = 0; t < MT; ++t) acc[t] = (float4_t){0.f, 0.f, 0.f, 0.f};
                    if constexpr (KS > 1) __syncthreads();         // partial sums read
                }
                crg += stride_rg;
            }
        }
    }
}

template <int MT, int U, int P, int WAVES, int KS>
hipError_t launch_mfma4_t(const uint16_t* X, int64_t M, const uint32_t* packed,
                          const uint16_t* scales, int64_t N, int64_t K, uint16_t* Y,
                          hipStream_t stream, int num_cu, int blocks_per_cu) {
    const size_t lds = (size_t)M * (K / 8 + 1) * 16 +
                       (size_t)(WAVES / KS) * (KS - 1) * MT * kWave * sizeof(float4_t);
    const int64_t total_rg = (N + 3) / 4;
    int64_t blocks;
    if constexpr (KS == 1) {
        // balanced persistent grid: every wave gets the same number of row groups
        const int64_t max_waves = (int64_t)num_cu * blocks_per_cu * WAVES;
        const int64_t per_wave = (total_rg + max_waves - 1) / max_waves;
        const int64_t waves = (total_rg + per_wave - 1) / per_wave;
        blocks = (waves + WAVES - 1) / WAVES;
    } else {
        // batches of WAVES / KS row groups, at most blocks_per_cu blocks per CU
        blocks = (total_rg + WAVES / KS - 1) / (WAVES / KS);
        if (blocks > (int64_t)num_cu * blocks_per_cu) blocks = (int64_t)num_cu * blocks_per_cu;
    }
    auto kern = gemv_mfma4_kernel<MT, U, P, WAVES, KS>;
    if (lds > 64 * 1024) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(WAVES * kWave), lds, stream, X, (int)M,
                       packed, scales, Y, (int)N, (int)K);
    return hipGetLastError();
}

hipError_t launch_gemv_mfma4(const uint16_t* X, int64_t M, const uint32_t* packed,
                             const uint16_t* scales, int64_t N, int64_t K, uint16_t* Y,
                             hipStream_t stream, int num_cu) {
    // Measured on gfx950 (4096 x 14336 and 14336 x 4096, M = 4): two loads
    // per step and two steps in flight; eight waves per block, one block per
    // compute unit, when x is small and there are row groups for eight waves
    // a CU; otherwise (the down projection: 1024 row groups, K = 14336) two
    // waves per row group, each taking every second step, which doubles the
    // waves a CU runs.
    const int64_t total_rg = (N + 3) / 4;
    const bool small_x = M * K * 2 <= 64 * 1024;
    if (small_x && total_rg >= (int64_t)8 * num_cu)
        return launch_mfma4_t<1, 2, 2, 8, 1>(X, M, packed, scales, N, K, Y, stream, num_cu, 1);
    return launch_mfma4_t<1, 2, 2, 8, 2>(X, M, packed, scales, N, K, Y, stream, num_cu,
                                         small_x ? 2 : 1);
}

}  // namespace w4a16

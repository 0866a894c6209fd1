// gemm_batched.hip — W4A16 GEMM for a few rows of X (batched decode,
// M <= 32) on the matrix cores.  Decode reads every weight once and is bound
// by memory ([BENCH] §二); a batch of M tokens reuses each weight M times, so
// up to a few dozen tokens the work is still one pass over the packed weights
// ([QUANT] dequantization s * q per group of 128).
//
// Y[m,n] = sum_g s[n,g] * sum_{k in g} q[n,k] * X[m,k]: the codes q are exact
// fp16 integers, v_mfma_f32_16x16x32_f16 forms the exact products q*x and
// sums one group in fp32, and the group's scale is applied with one fp32 FMA
// per output (as the GEMV applies it per group).
//
// Work split.  Block b owns the contiguous weight rows [b*R, b*R + R) and
// walks all of K; it holds the accumulators of all its rows in registers, so
// X is read once per block and weights once in total.  Its waves form a
// WR x WKS grid: wave (wr, ws) owns the 16-row tiles wr, wr + WR, ... (TN of
// them) and the groups ws, ws + WKS, ... of every chunk of K.  X is staged
// chunk by chunk into LDS (double buffered, paired order of codes_word,
// rows padded by 16 bytes so the 16 rows of a fragment read hit distinct
// banks) together with the block's scales of the chunk (its rows times the
// chunk's groups, a few KB: one scale load per lane and group would cost
// about as much as the code load it belongs to); chunk c + 1 is loaded into
// registers while chunk c is used, one barrier per chunk.  Weights never
// pass through LDS: lane (n = l%16, j = l/16) loads 16 bytes of row n per
// group (words 4j..4j+3, the B operand of the four k-steps) through a ring
// of Q register slots, Q - 1 groups ahead of use, across chunk boundaries.
// The loop body is unrolled over whole chunks and ring turns, so every load
// sits at a fixed place and each wait covers exactly the load it needs
// (loads complete in order; a wait placed for a load issued before a
// data-dependent branch would also wait for everything issued after it).
// At the end the WKS partial tiles of each row tile are added through LDS in
// a fixed order, so results do not depend on timing.
//
// Operand mapping of v_mfma_f32_16x16x32_f16 (lane l, j = l/16):
//   A (16 x 32): X row l%16, eight k of slot j
//   B (32 x 16): weight row l%16, the same eight k
//   D (16 x 16): X rows 4j..4j+3 of weight row l%16
// Rows past M read a clamped row of the staged X (their outputs are never
// stored); rows past the block's range and k past K read 0 through buffer
// bounds, and groups past K are skipped.
//
// Asymmetric weights (ASYM, [QUANT] sub-section 2: w = s (n - z), nibble n
// in [0, 15], an int16 zero point z per row and group): the zero points are
// staged beside the scales, the B operand holds the exact codes n - zc
// (codes_word_zp, zc = z clamped to +-1000), and a group with |z| > 1000
// adds s (zc - z) times the group's activation sums, which one more MFMA
// per k-step against a B of ones forms (only in waves that hold such a
// group), as the tiled kernel does.
#include "w4a16_device.h"
#include "w4a16_launch.h"

namespace w4a16 {

namespace {
constexpr int kBatchedXVecs = 8;                    // staged 16-byte vectors per thread and chunk
constexpr int kBatchedScales = 4;                   // staged scales per thread and chunk
}  // namespace

// MT: 16-row tiles of X; TN: 16-row weight tiles per wave; WR x WKS: wave
// grid; GPW: groups per wave and chunk (chunk = GPW * WKS groups); Q: weight
// ring slots (power of two).
template <int MT, int TN, int WR, int WKS, int GPW, int Q, bool ASYM>
__global__ __launch_bounds__(WR * WKS * kWave) void gemm_batched_kernel(
    const uint16_t* __restrict__ X, int M, const uint32_t* __restrict__ packed,
    const uint16_t* __restrict__ scales, const int16_t* __restrict__ zeros,
    uint16_t* __restrict__ Y, int N, int K, int rows_per_block) {
    constexpr int NT = WR * WKS * kWave;
    constexpr int P = Q - 1;                          // groups in flight ahead of use
    constexpr int U = Q > GPW ? Q / GPW : 1;          // chunks per unrolled body
    constexpr int IB = U * GPW;                       // groups per body, a multiple of Q
    static_assert(IB % Q == 0, "ring slots must divide the body");
    constexpr int GC = GPW * WKS;                     // groups per chunk
    constexpr int KC = GC * kGroup;                   // chunk width in k
    constexpr int CBLK = KC / 8;                      // 8-element blocks per staged row
    constexpr int XSTRIDE = CBLK + 1;                 // 16-byte pad per row
    constexpr int XV = kBatchedXVecs;
    constexpr int SV = kBatchedScales;
    constexpr int SROWS = 16 * WR * TN;               // rows covered by the waves' tiles
    constexpr int SBUF = SROWS * GC;                  // staged scales per buffer
    static_assert(16 * MT * CBLK <= XV * NT, "X chunk exceeds the staging registers");
    static_assert(SBUF <= SV * NT, "scale chunk exceeds the staging registers");
    extern __shared__ uint4 lds[];                    // 2 x [xrows][XSTRIDE] paired X,
                                                      // then 2 x [SROWS][GC] scales
                                                      // (and as many zero points)

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int wr = wave % WR;
    const int ws = wave / WR;
    const int l16 = lane & 15;
    const int j = lane >> 4;
    const int r0 = blockIdx.x * rows_per_block;
    const int nrows = min(N - r0, rows_per_block);    // > 0: the grid covers N exactly
    const int xrows = min(M, 16 * MT);
    const int ngroups = K >> 7;
    const int nchunks = (ngroups + GC - 1) / GC;
    const int xbuf = xrows * XSTRIDE;
    const int xtotal = xrows * CBLK;
    uint16_t* const slds = reinterpret_cast<uint16_t*>(lds + 2 * xbuf);
    int16_t* const zlds = reinterpret_cast<int16_t*>(slds + 2 * SBUF);
    const int c_first = (int)(blockIdx.x % (unsigned)nchunks);
    const uint32_t wrow = (uint32_t)K / 2, srow = (uint32_t)K / 64;
    const uint32_t xbytes = (uint32_t)M * (uint32_t)K * 2u;
    const uint32_t sbytes = (uint32_t)nrows * srow;
    const CodeConsts kcst = code_consts();

    typedef unsigned v4u __attribute__((ext_vector_type(4)));
    const __amdgpu_buffer_rsrc_t wr_live = buffer_rsrc(
        reinterpret_cast<const char*>(packed) + (size_t)r0 * wrow, (uint64_t)nrows * wrow);
    const __amdgpu_buffer_rsrc_t sr = buffer_rsrc(
        reinterpret_cast<const char*>(scales) + (size_t)r0 * srow, sbytes);
    const __amdgpu_buffer_rsrc_t zr =
        ASYM ? buffer_rsrc(reinterpret_cast<const char*>(zeros) + (size_t)r0 * srow, sbytes) : sr;
    const __amdgpu_buffer_rsrc_t empty = buffer_rsrc(packed, 0);
    const __amdgpu_buffer_rsrc_t xr = buffer_rsrc(X, xbytes);

    // chunk sequence number -> chunk index (blocks start at different chunks
    // so that they do not all read the same X lines at once)
    auto chunk_of = [&](int cc) {
        const int c = c_first + cc;
        return c >= nchunks ? c - nchunks : c;
    };

    // ---- X and scale chunks: global -> registers -> LDS.  Every chunk
    // start runs the same code (chunks past the end load nothing), so the
    // compiler knows at every weight wait exactly which loads are younger.
    v4u xv[XV];
    uint32_t sv[SV], zv[SV];
    auto x_load = [&](int cc) {
        const bool live = cc < nchunks;
        const int c = chunk_of(cc);
#pragma unroll
        for (int i = 0; i < XV; ++i) {
            const int e = threadIdx.x + i * NT;
            const int row = e / CBLK;
            const int k = c * KC + (e % CBLK) * 8;
            const uint32_t off = (live && e < xtotal && k < K)
                                     ? ((uint32_t)row * (uint32_t)K + (uint32_t)k) * 2u
                                     : xbytes;
            xv[i] = __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < SV; ++i) {
            const int e = threadIdx.x + i * NT;
            const uint32_t off = (live && e < SBUF)
                                     ? (uint32_t)(e / GC) * srow + (uint32_t)(c * GC + e % GC) * 2u
                                     : sbytes;
            sv[i] = __builtin_amdgcn_raw_buffer_load_b16(sr, off, 0, 0);
            zv[i] = ASYM ? __builtin_amdgcn_raw_buffer_load_b16(zr, off, 0, 0) : 0u;
        }
    };
    auto x_store = [&](int buf) {
#pragma unroll
        for (int i = 0; i < XV; ++i) {
            const int e = threadIdx.x + i * NT;
            if (e < xtotal)
                lds[buf * xbuf + (e / CBLK) * XSTRIDE + e % CBLK] =
                    pair_block(xv[i].x, xv[i].y, xv[i].z, xv[i].w);
        }
#pragma unroll
        for (int i = 0; i < SV; ++i) {
            const int e = threadIdx.x + i * NT;
            if (e < SBUF) {
                slds[buf * SBUF + e] = (uint16_t)sv[i];
                if constexpr (ASYM) zlds[buf * SBUF + e] = (int16_t)(uint16_t)zv[i];
            }
        }
    };

    // ---- weight ring: group t + P is loaded before group t is used
    struct Slot {
        v4u w[TN];
    };
    int lcc = 0, li = 0;                              // load cursor: chunk sequence, group in chunk
    auto load = [&](Slot& sl) {
        const int g = chunk_of(lcc) * GC + ws + WKS * li;
        const bool live = lcc < nchunks && g < ngroups;
        const __amdgpu_buffer_rsrc_t w = live ? wr_live : empty;
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
            const uint32_t row = (uint32_t)(16 * (wr + WR * tn) + l16);
            sl.w[tn] = __builtin_amdgcn_raw_buffer_load_b128(w, row * wrow + g * 64 + j * 16, 0,
                                                             kStreamLoad);
        }
        if (++li == GPW) {
            li = 0;
            ++lcc;
        }
    };

    x_load(0);
    Slot ring[Q];
#pragma unroll
    for (int i = 0; i < P; ++i) load(ring[i]);

    float4_t acc[MT][TN];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) acc[mt][tn] = (float4_t){0.f, 0.f, 0.f, 0.f};
    int xrow_off[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) xrow_off[mt] = min(mt * 16 + l16, xrows - 1) * XSTRIDE;

    for (int cb = 0; cb < nchunks; cb += U) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int cc = cb + u;
            const int buf = cc & 1;
            // buffer cc & 1 was last read in chunk cc - 2, finished before the
            // barrier of chunk cc - 1
            x_store(buf);
            __syncthreads();
            x_load(cc + 1);
            const int cbase = chunk_of(cc) * GC;
#pragma unroll
            for (int i = 0; i < GPW; ++i) {
                const int sidx = u * GPW + i;         // static slot position in the body
                load(ring[(sidx + P) % Q]);
                const int gl = ws + WKS * i;
                if (cc < nchunks && cbase + gl < ngroups) {   // wave-uniform
                    const Slot& sl = ring[sidx % Q];
                    const uint4* xb = lds + buf * xbuf + gl * 16 + 4 * j;
                    ZeroBias zb[TN];
                    bool wide = false;
                    if constexpr (ASYM) {
#pragma unroll
                        for (int tn = 0; tn < TN; ++tn) {
                            const int z = zlds[buf * SBUF + (16 * (wr + WR * tn) + l16) * GC + gl];
                            zb[tn] = zero_bias(z);
                            wide |= zb[tn].zc != z;
                        }
                    }
                    float4_t d[MT][TN];
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk) {
                        half8_t bq[TN];
#pragma unroll
                        for (int tn = 0; tn < TN; ++tn) {
                            half2_t q[4];
                            if constexpr (ASYM)
                                codes_word_zp(sl.w[tn][kk], kcst, zb[tn], q);
                            else
                                codes_word(sl.w[tn][kk], kcst, q);
                            bq[tn] = (half8_t){q[0].x, q[0].y, q[1].x, q[1].y,
                                               q[2].x, q[2].y, q[3].x, q[3].y};
                        }
#pragma unroll
                        for (int mt = 0; mt < MT; ++mt) {
                            const half8_t af = __builtin_bit_cast(half8_t, xb[xrow_off[mt] + kk]);
#pragma unroll
                            for (int tn = 0; tn < TN; ++tn)
                                d[mt][tn] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                                    af, bq[tn],
                                    kk == 0 ? (float4_t){0.f, 0.f, 0.f, 0.f} : d[mt][tn], 0, 0,
                                    0);
                        }
                    }
#pragma unroll
                    for (int tn = 0; tn < TN; ++tn) {
                        const float sc = f16_bits_to_f32(
                            slds[buf * SBUF + (16 * (wr + WR * tn) + l16) * GC + gl]);
#pragma unroll
                        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                            for (int r = 0; r < 4; ++r)
                                acc[mt][tn][r] = fmaf(sc, d[mt][tn][r], acc[mt][tn][r]);
                    }
                    if constexpr (ASYM) {
                        if (__any(wide)) {
                            // activation sums of the group's 128 k for each X row
                            const _Float16 one = (_Float16)1.0f;
                            const half8_t ones = {one, one, one, one, one, one, one, one};
                            float4_t xs[MT];
#pragma unroll
                            for (int kk = 0; kk < 4; ++kk)
#pragma unroll
                                for (int mt = 0; mt < MT; ++mt)
                                    xs[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                                        __builtin_bit_cast(half8_t, xb[xrow_off[mt] + kk]), ones,
                                        kk == 0 ? (float4_t){0.f, 0.f, 0.f, 0.f} : xs[mt], 0, 0,
                                        0);
#pragma unroll
                            for (int tn = 0; tn < TN; ++tn) {
                                const int row = 16 * (wr + WR * tn) + l16;
                                const int z = zlds[buf * SBUF + row * GC + gl];
                                const float cf =
                                    f16_bits_to_f32(slds[buf * SBUF + row * GC + gl]) *
                                    (float)(zb[tn].zc - z);
#pragma unroll
                                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                                    for (int r = 0; r < 4; ++r)
                                        acc[mt][tn][r] = fmaf(cf, xs[mt][r], acc[mt][tn][r]);
                            }
                        }
                    }
                }
            }
        }
    }

    // ---- sum the WKS partial tiles of each row tile in a fixed order
    if constexpr (WKS > 1) {
        float4_t* red = reinterpret_cast<float4_t*>(lds);
        __syncthreads();                              // X buffers no longer read
        if (ws > 0) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int tn = 0; tn < TN; ++tn)
                    red[((((ws - 1) * WR + wr) * MT + mt) * TN + tn) * kWave + lane] =
                        acc[mt][tn];
        }
        __syncthreads();
        if (ws > 0) return;
#pragma unroll
        for (int w = 1; w < WKS; ++w)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int tn = 0; tn < TN; ++tn)
                    acc[mt][tn] += red[((((w - 1) * WR + wr) * MT + mt) * TN + tn) * kWave + lane];
    }
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
        const int nl = 16 * (wr + WR * tn) + l16;
        if (nl >= nrows) continue;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = mt * 16 + 4 * j + r;
                if (m < M) Y[(size_t)m * N + r0 + nl] = f32_to_f16_bits(acc[mt][tn][r]);
            }
    }
}

template <int MT, int TN, int WR, int WKS, int GPW, int Q, bool ASYM>
hipError_t launch_batched_t(const uint16_t* X, int64_t M, const uint32_t* packed,
                            const uint16_t* scales, const int16_t* zeros, int64_t N, int64_t K,
                            uint16_t* Y, hipStream_t stream, int64_t rows_per_block) {
    constexpr int NT = WR * WKS * kWave;
    constexpr int64_t KC = (int64_t)GPW * WKS * kGroup;
    const int64_t xrows = M < 16 * MT ? M : 16 * MT;
    if (rows_per_block > 16 * WR * TN || M > 16 * MT) return hipErrorInvalidValue;
    const size_t x_lds = (size_t)2 * xrows * (KC / 8 + 1) * 16 +
                         (size_t)(ASYM ? 2 : 1) * 2 * (16 * WR * TN) * (KC / kGroup) * 2;
    const size_t red_lds = (size_t)(WKS - 1) * WR * MT * TN * kWave * sizeof(float4_t);
    const size_t lds = x_lds > red_lds ? x_lds : red_lds;
    if (lds > 64 * 1024) {
        const hipError_t e = hipFuncSetAttribute(
            reinterpret_cast<const void*>(gemm_batched_kernel<MT, TN, WR, WKS, GPW, Q, ASYM>),
            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    const int64_t blocks = (N + rows_per_block - 1) / rows_per_block;
    hipLaunchKernelGGL((gemm_batched_kernel<MT, TN, WR, WKS, GPW, Q, ASYM>),
                       dim3((unsigned)blocks), dim3(NT), lds, stream, X, (int)M, packed, scales,
                       zeros, Y, (int)N, (int)K, (int)rows_per_block);
    return hipGetLastError();
}

// Chunks: 2048 k for up to 16 rows of X, 1024 k for up to 32 (two staged
// copies of X and scales, 130-136 KB of LDS).
// Measured on gfx950 (4096 x 6144 .. 4096 x 28672 and 14336 x 4096, M = 8,
// 16, 32): two 16-row tiles per wave with a 2 x 4 wave grid for 17..64 rows a
// block, four tiles for more, eight waves over K for at most 16 rows (the
// down projection); four ring slots, two for the widest tiles.
template <int MT, bool ASYM>
hipError_t launch_batched_m(const uint16_t* X, int64_t M, const uint32_t* packed,
                            const uint16_t* scales, const int16_t* zeros, int64_t N, int64_t K,
                            uint16_t* Y, hipStream_t stream, int num_cu) {
    // one block per compute unit, rows split evenly; at most 128 rows a block
    int64_t rpb = (N + num_cu - 1) / num_cu;
    if (rpb > 128) rpb = 128;
    const int64_t tiles = (rpb + 15) / 16;
    constexpr int G = 16 / MT;                        // groups per chunk
    if (tiles <= 1)
        return launch_batched_t<MT, 1, 1, 8, G / 8, 4 / MT, ASYM>(X, M, packed, scales, zeros, N,
                                                                  K, Y, stream, rpb);
    if (tiles <= 2)
        return launch_batched_t<MT, 2, 1, 8, G / 8, 4, ASYM>(X, M, packed, scales, zeros, N, K,
                                                             Y, stream, rpb);
    if (tiles <= 4)
        return launch_batched_t<MT, 2, 2, 4, G / 4, 4, ASYM>(X, M, packed, scales, zeros, N, K,
                                                             Y, stream, rpb);
    return launch_batched_t<MT, 4, 2, 4, G / 4, 2, ASYM>(X, M, packed, scales, zeros, N, K, Y,
                                                         stream, rpb);
}

hipError_t launch_gemm_batched(const uint16_t* X, int64_t M, const uint32_t* packed,
                               const uint16_t* scales, int64_t N, int64_t K, uint16_t* Y,
                               hipStream_t stream, int num_cu) {
    if (M <= 16)
        return launch_batched_m<1, false>(X, M, packed, scales, nullptr, N, K, Y, stream, num_cu);
    return launch_batched_m<2, false>(X, M, packed, scales, nullptr, N, K, Y, stream, num_cu);
}

hipError_t launch_gemm_batched_asym(const uint16_t* X, int64_t M, const uint32_t* packed,
                                    const uint16_t* scales, const int16_t* zeros, int64_t N,
                                    int64_t K, uint16_t* Y, hipStream_t stream, int num_cu) {
    if (M <= 16)
        return launch_batched_m<1, true>(X, M, packed, scales, zeros, N, K, Y, stream, num_cu);
    return launch_batched_m<2, true>(X, M, packed, scales, zeros, N, K, Y, stream, num_cu);
}

}  // namespace w4a16

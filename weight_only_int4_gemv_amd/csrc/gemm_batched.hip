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
// Split K (SPLIT, batched decode with a caller workspace): when a block
// would own only a few rows of a long-K matrix (the down projection), X is
// the bulk of what each block reads (every block needs all of X for its
// rows).  Block (b, k) then owns more rows and only the groups of K-slice k:
// X per block shrinks by the number of slices.  Each block stores its fp32
// partial tile to the workspace with device-coherent stores, waits for them
// and counts itself on its row block's counter; the block that counts last
// adds the slices' partials in slice order (the same order whichever block
// is last, so results do not depend on timing), writes Y and returns the
// counter to zero.  No block ever waits for another.
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
constexpr int kCoherent = 16;                       // cache policy: coherent at device scope (sc1)
}  // namespace

// MT: 16-row tiles of X; TN: 16-row weight tiles per wave; WR x WKS: wave
// grid; GPW: groups per wave and chunk (chunk = GPW * WKS groups); Q: weight
// ring slots (power of two).
template <int MT, int TN, int WR, int WKS, int GPW, int Q, bool ASYM, bool SPLIT>
__global__ __launch_bounds__(WR * WKS * kWave) void gemm_batched_kernel(
    const uint16_t* __restrict__ X, int M, const uint32_t* __restrict__ packed,
    const uint16_t* __restrict__ scales, const int16_t* __restrict__ zeros,
    uint16_t* __restrict__ Y, int N, int K, int rows_per_block, int ksplit, int gps,
    uint32_t* __restrict__ counters, float4_t* __restrict__ partials) {
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
    // row block and K slice (groups [g_lo, g_lo + ngroups) of the row)
    const int rb = SPLIT ? (int)(blockIdx.x / (unsigned)ksplit) : (int)blockIdx.x;
    const int ks = SPLIT ? (int)(blockIdx.x - (unsigned)rb * (unsigned)ksplit) : 0;
    const int r0 = rb * rows_per_block;
    const int nrows = min(N - r0, rows_per_block);    // > 0: the grid covers N exactly
    const int xrows = min(M, 16 * MT);
    const int g_lo = SPLIT ? ks * gps : 0;
    const int ngroups = SPLIT ? min(K >> 7, g_lo + gps) - g_lo : (K >> 7);   // > 0
    const int k_lo = g_lo * kGroup, k_hi = k_lo + ngroups * kGroup;
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
            const int k = k_lo + c * KC + (e % CBLK) * 8;
            const uint32_t off = (live && e < xtotal && k < k_hi)
                                     ? ((uint32_t)row * (uint32_t)K + (uint32_t)k) * 2u
                                     : xbytes;
            xv[i] = __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < SV; ++i) {
            const int e = threadIdx.x + i * NT;
            const uint32_t off = (live && e < SBUF)
                                     ? (uint32_t)(e / GC) * srow +
                                           (uint32_t)(g_lo + c * GC + e % GC) * 2u
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
        const int gr = chunk_of(lcc) * GC + ws + WKS * li;    // group in the slice
        const bool live = lcc < nchunks && gr < ngroups;
        const int g = g_lo + gr;
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
    if constexpr (SPLIT) {
        // partial tile of this slice -> workspace, in the lanes' own layout
        // (the reducing block reads it back the same way)
        __shared__ uint32_t last_flag;
        constexpr int PT = WR * TN * MT * kWave;          // float4 per block partial
        const __amdgpu_buffer_rsrc_t pr = buffer_rsrc(
            partials + (size_t)rb * ksplit * PT, (uint64_t)ksplit * PT * sizeof(float4_t));
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const uint32_t off =
                    (uint32_t)((ks * PT + ((wr * TN + tn) * MT + mt) * kWave + lane) * 16);
                const v4u v = {__float_as_uint(acc[mt][tn][0]), __float_as_uint(acc[mt][tn][1]),
                               __float_as_uint(acc[mt][tn][2]), __float_as_uint(acc[mt][tn][3])};
                __builtin_amdgcn_raw_buffer_store_b128(v, pr, off, 0, kCoherent);
            }
        __builtin_amdgcn_s_waitcnt(0x0F70);               // vmcnt(0): stores complete
        __syncthreads();                                  // every wave's stores are complete
        if (threadIdx.x == 0)
            last_flag = __hip_atomic_fetch_add(&counters[rb], 1u, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        if (last_flag != (uint32_t)(ksplit - 1)) return;
        // the last slice of this row block: sum every slice in slice order
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc[mt][tn] = (float4_t){0.f, 0.f, 0.f, 0.f};
        for (int sl = 0; sl < ksplit; ++sl) {
#pragma unroll
            for (int tn = 0; tn < TN; ++tn)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const uint32_t off =
                        (uint32_t)((sl * PT + ((wr * TN + tn) * MT + mt) * kWave + lane) * 16);
                    const v4u v = __builtin_amdgcn_raw_buffer_load_b128(pr, off, 0, kCoherent);
                    acc[mt][tn] += (float4_t){__uint_as_float(v.x), __uint_as_float(v.y),
                                              __uint_as_float(v.z), __uint_as_float(v.w)};
                }
        }
        if (threadIdx.x == 0)
            __hip_atomic_store(&counters[rb], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

namespace {

template <int MT, int TN, int WR, int WKS, int GPW, int Q, bool ASYM, bool SPLIT = false>
hipError_t launch_batched_t(const uint16_t* X, int64_t M, const uint32_t* packed,
                            const uint16_t* scales, const int16_t* zeros, int64_t N, int64_t K,
                            uint16_t* Y, hipStream_t stream, int64_t rows_per_block,
                            const BatchedSplit* split = nullptr) {
    constexpr int NT = WR * WKS * kWave;
    constexpr int64_t KC = (int64_t)GPW * WKS * kGroup;
    const int64_t xrows = M < 16 * MT ? M : 16 * MT;
    if (rows_per_block > 16 * WR * TN || M > 16 * MT) return hipErrorInvalidValue;
    if (SPLIT && (split == nullptr || split->rows_per_block != rows_per_block ||
                  split->tile_rows != 16 * WR * TN || split->tile_m != 16 * MT))
        return hipErrorInvalidValue;
    const size_t x_lds = (size_t)2 * xrows * (KC / 8 + 1) * 16 +
                         (size_t)(ASYM ? 2 : 1) * 2 * (16 * WR * TN) * (KC / kGroup) * 2;
    const size_t red_lds = (size_t)(WKS - 1) * WR * MT * TN * kWave * sizeof(float4_t);
    const size_t lds = x_lds > red_lds ? x_lds : red_lds;
    auto kern = gemm_batched_kernel<MT, TN, WR, WKS, GPW, Q, ASYM, SPLIT>;
    if (lds > 64 * 1024) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 (int)lds);
        if (e != hipSuccess) return e;
    }
    const int64_t row_blocks = (N + rows_per_block - 1) / rows_per_block;
    const int ksplit = SPLIT ? split->ksplit : 1;
    const int gps = SPLIT ? split->groups_per_slice : 0;
    hipLaunchKernelGGL(kern, dim3((unsigned)(row_blocks * ksplit)), dim3(NT), lds, stream, X,
                       (int)M, packed, scales, zeros, Y, (int)N, (int)K, (int)rows_per_block,
                       ksplit, gps, SPLIT ? split->counters : nullptr,
                       SPLIT ? reinterpret_cast<float4_t*>(split->partials) : nullptr);
    return hipGetLastError();
}

// Chunks: 2048 k for up to 16 rows of X, 1024 k for up to 32 (two staged
// copies of X and scales, 130-136 KB of LDS).
// Measured on gfx950 (4096 x 6144 .. 4096 x 28672 and 14336 x 4096, M = 8,
// 16, 32): two 16-row tiles per wave with a 2 x 4 wave grid for 17..64 rows a
// block, four tiles for more, eight waves over K for at most 16 rows (the
// down projection); four ring slots, two for the widest tiles.
template <int MT, bool ASYM, bool SPLIT = false>
hipError_t launch_batched_rows(const uint16_t* X, int64_t M, const uint32_t* packed,
                               const uint16_t* scales, const int16_t* zeros, int64_t N,
                               int64_t K, uint16_t* Y, hipStream_t stream, int64_t rpb,
                               const BatchedSplit* split = nullptr) {
    const int64_t tiles = (rpb + 15) / 16;
    constexpr int G = 16 / MT;                        // groups per chunk
    if (tiles <= 1)
        return launch_batched_t<MT, 1, 1, 8, G / 8, 4 / MT, ASYM, SPLIT>(
            X, M, packed, scales, zeros, N, K, Y, stream, rpb, split);
    if (tiles <= 2)
        return launch_batched_t<MT, 2, 1, 8, G / 8, 4, ASYM, SPLIT>(
            X, M, packed, scales, zeros, N, K, Y, stream, rpb, split);
    if (tiles <= 4)
        return launch_batched_t<MT, 2, 2, 4, G / 4, 4, ASYM, SPLIT>(
            X, M, packed, scales, zeros, N, K, Y, stream, rpb, split);
    return launch_batched_t<MT, 4, 2, 4, G / 4, 2, ASYM, SPLIT>(X, M, packed, scales, zeros, N,
                                                                K, Y, stream, rpb, split);
}

template <int MT, bool ASYM>
hipError_t launch_batched_m(const uint16_t* X, int64_t M, const uint32_t* packed,
                            const uint16_t* scales, const int16_t* zeros, int64_t N, int64_t K,
                            uint16_t* Y, hipStream_t stream, int num_cu) {
    // one block per compute unit, rows split evenly; at most 128 rows a block
    int64_t rpb = (N + num_cu - 1) / num_cu;
    if (rpb > 128) rpb = 128;
    return launch_batched_rows<MT, ASYM>(X, M, packed, scales, zeros, N, K, Y, stream, rpb);
}

// The 16-row tiles a block of `rows` rows is launched with (the wave grid of
// launch_batched_rows): 16, 32, 64 or 128 rows.
int64_t batched_tile_rows(int64_t rows) {
    const int64_t tiles = (rows + 15) / 16;
    return tiles <= 1 ? 16 : tiles <= 2 ? 32 : tiles <= 4 ? 64 : 128;
}

}  // namespace

BatchedSplit plan_batched_split(int64_t M, int64_t N, int64_t K, int num_cu, int64_t rows,
                                int ksplit) {
    BatchedSplit p{};
    p.ksplit = 1;
    const int64_t ngroups = K / kGroup;
    if (M < 1 || M > kBatchedMaxM || N < 1 || ngroups < 2 || K > kBatchedMaxK) return p;
    if (rows <= 0 || ksplit <= 0) {
        // Measured on gfx950 (14336 x 4096 and 4096 x 14336, M = 8..32):
        // split only rows shorter than the K they walk (N < 2K with at most
        // N / CUs rows a block): 64-row blocks and as many K slices as keep
        // one block per compute unit.
        const int64_t per_cu = (N + num_cu - 1) / num_cu;
        if (K < 2 * N || per_cu > 32) return p;
        rows = 64;
        const int64_t row_blocks = (N + rows - 1) / rows;
        ksplit = (int)(num_cu / row_blocks);          // at most one block per CU
    }
    if (rows > 128) rows = 128;
    if (ksplit > ngroups) ksplit = (int)ngroups;
    const int64_t gps = (ngroups + ksplit - 1) / ksplit;
    ksplit = (int)((ngroups + gps - 1) / gps);        // every slice holds a group
    const int64_t row_blocks = (N + rows - 1) / rows;
    if (ksplit < 2 || row_blocks > kBatchedSplitCounters) return p;
    p.ksplit = ksplit;
    p.groups_per_slice = (int)gps;
    p.rows_per_block = (int)rows;
    p.tile_rows = (int)batched_tile_rows(rows);
    p.tile_m = M <= 16 ? 16 : 32;
    // the counters always take the same first bytes of the workspace, so a
    // workspace used for several shapes never has partials where another
    // shape's counters are
    p.counter_bytes = (size_t)kBatchedSplitCounters * 4;
    p.workspace_bytes = p.counter_bytes +
                        (size_t)row_blocks * ksplit * p.tile_rows * p.tile_m * sizeof(float);
    return p;
}

hipError_t launch_gemm_batched_split(const uint16_t* X, int64_t M, const uint32_t* packed,
                                     const uint16_t* scales, int64_t N, int64_t K, uint16_t* Y,
                                     hipStream_t stream, const BatchedSplit& plan,
                                     void* workspace) {
    if (plan.ksplit < 2) return hipErrorInvalidValue;
    BatchedSplit p = plan;
    p.counters = static_cast<uint32_t*>(workspace);
    p.partials = static_cast<char*>(workspace) + plan.counter_bytes;
    if (M <= 16)
        return launch_batched_rows<1, false, true>(X, M, packed, scales, nullptr, N, K, Y, stream,
                                                   p.rows_per_block, &p);
    return launch_batched_rows<2, false, true>(X, M, packed, scales, nullptr, N, K, Y, stream,
                                               p.rows_per_block, &p);
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

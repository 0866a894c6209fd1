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
//
// Asymmetric INT4 ([QUANT] sub-section 2, asymmetric equations: w = s (n - z)
// with the nibble n in [0, 15] and an integer zero point z per group): the
// codes are formed as n - zc, exact fp16 integers, with zc = clamp(z, -1000,
// 1000) folded into the two bias constants of the code trick, so the products
// stay exact; a group with |z| > 1000 (one-signed with a narrow range, where
// every |n - z| > 985) adds (zc - z) * sum(x over the chunk).
#include <atomic>

#include "w4a16_device.h"
#include "w4a16_launch.h"

namespace w4a16 {

namespace {

// The 8 activations of row m at positions col0 .. col0+7 of the weight's
// column order.  Without perm they are X[m, col0 .. col0+7]; with perm (the
// act-order layout, [QUANT] GPTQ section: columns quantized and stored in
// the order perm, activations permuted the same way at inference) they are
// X[m, perm[col0 + i]], and an index outside [0, K) reads as 0.
__device__ __forceinline__ uint4 x_block(const uint16_t* __restrict__ X, int m, int K, int col0,
                                         const int* __restrict__ perm) {
    const uint16_t* row = X + (size_t)m * K;
    if (perm == nullptr) return reinterpret_cast<const uint4*>(row + col0)[0];
    const int4 p0 = reinterpret_cast<const int4*>(perm + col0)[0];
    const int4 p1 = reinterpret_cast<const int4*>(perm + col0)[1];
    const int idx[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
    uint32_t h[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) h[i] = (uint32_t)idx[i] < (uint32_t)K ? row[idx[i]] : 0u;
    return make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                      h[6] | (h[7] << 16));
}

// Stage activation rows [0, M) x elements [k0, k0 + ks) into LDS:
//   xs[m * (ks/8) + b] = paired 8-element block b of the slice.
__device__ __forceinline__ void stage_activations(const uint16_t* __restrict__ X, int M, int K,
                                                  int k0, int ks, uint4* xs,
                                                  const int* __restrict__ perm) {
    const int nblk = ks >> 3;
    const int total = M * nblk;
    constexpr int B = 4;  // loads issued before the first store
    for (int i0 = threadIdx.x; i0 < total; i0 += B * blockDim.x) {
        uint4 v[B];
#pragma unroll
        for (int j = 0; j < B; ++j) {
            const int i = i0 + j * blockDim.x;
            if (i < total) {
                const int m = i / nblk;
                v[j] = x_block(X, m, K, k0 + (i - m * nblk) * 8, perm);
            }
        }
#pragma unroll
        for (int j = 0; j < B; ++j) {
            const int i = i0 + j * blockDim.x;
            if (i < total) xs[i] = pair_block(v[j].x, v[j].y, v[j].z, v[j].w);
        }
    }
}

// acc += sum of the 8 products x * (n - zc) of one packed word (exact fp16
// codes from codes_word_zp, exact products in v_dot2_f32_f16).
__device__ __forceinline__ float dot_word_zp(uint32_t w, const uint4& xp, float acc,
                                             const CodeConsts& k, const ZeroBias& b) {
    half2_t q[4];
    codes_word_zp(w, k, b, q);
    acc = __builtin_amdgcn_fdot2(q[0], as_h2(xp.x), acc, false);
    acc = __builtin_amdgcn_fdot2(q[1], as_h2(xp.y), acc, false);
    acc = __builtin_amdgcn_fdot2(q[2], as_h2(xp.z), acc, false);
    acc = __builtin_amdgcn_fdot2(q[3], as_h2(xp.w), acc, false);
    return acc;
}

// sum_k x_k * (n_k - z) over one 16-byte chunk of 32 codes (activations
// x0..x3 in the paired order).  Symmetric weights (ASYM false) have
// n_k - 8 instead and ignore z.
template <bool ASYM>
__device__ __forceinline__ float chunk_dot(const uint4& w, const uint4& x0, const uint4& x1,
                                           const uint4& x2, const uint4& x3, int z,
                                           const CodeConsts& kc) {
    if constexpr (!ASYM) {
        float part = dot_word(w.x, x0, 0.0f, kc);
        part = dot_word(w.y, x1, part, kc);
        part = dot_word(w.z, x2, part, kc);
        return dot_word(w.w, x3, part, kc);
    } else {
        const ZeroBias b = zero_bias(z);
        float part = dot_word_zp(w.x, x0, 0.0f, kc, b);
        part = dot_word_zp(w.y, x1, part, kc, b);
        part = dot_word_zp(w.z, x2, part, kc, b);
        part = dot_word_zp(w.w, x3, part, kc, b);
        if (b.zc != z) {
            // sum of the chunk's 32 activations, each exact in fp32
            const half2_t one = {(_Float16)1.0f, (_Float16)1.0f};
            float xs = 0.0f;
            const uint32_t xv[16] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w,
                                     x2.x, x2.y, x2.z, x2.w, x3.x, x3.y, x3.z, x3.w};
#pragma unroll
            for (int i = 0; i < 16; ++i) xs = __builtin_amdgcn_fdot2(one, as_h2(xv[i]), xs, false);
            part = fmaf((float)(b.zc - z), xs, part);
        }
        return part;
    }
}

}  // namespace

// MMAX: activation rows handled (M <= MMAX at run time).  R: weight rows per
// wave.  U: chunk steps loaded ahead.  WAVES: waves per block.  ASYM: the
// asymmetric layout, one int16 zero point per group in `zeros` (laid out like
// the scales); NULL and unused otherwise.
template <int MMAX, int R, int U, int WAVES, bool ASYM>
__global__ __launch_bounds__(WAVES * kWave) void gemv_kernel(
    const uint16_t* __restrict__ X, int M, const uint4* __restrict__ packed,
    const uint16_t* __restrict__ scales, const int16_t* __restrict__ zeros,
    uint16_t* __restrict__ Y, int N, int K, int kslice, int gshift,
    const int* __restrict__ perm) {
    extern __shared__ uint4 lds[];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int nchunks = K >> 5;                   // 16-byte chunks per weight row
    const int ngroups = scales_per_row(K, gshift);  // scales per weight row (2^gshift chunks each)
    const int row0 = (blockIdx.x * WAVES + wave) * R;

    size_t wrow[R], srow[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int row = min(row0 + r, N - 1);  // tail rows re-read row N-1, never stored
        wrow[r] = (size_t)row * nchunks;
        srow[r] = (size_t)row * ngroups;
    }

    const CodeConsts kc = code_consts();
    float acc[MMAX][R];
#pragma unroll
    for (int m = 0; m < MMAX; ++m)
#pragma unroll
        for (int r = 0; r < R; ++r) acc[m][r] = 0.0f;

    for (int k0 = 0; k0 < K; k0 += kslice) {
        const int ks = min(kslice, K - k0);
        const int c0 = k0 >> 5;          // first chunk of the slice
        const int nch = ks >> 5;
        const int nsteps = (nch + kWave - 1) / kWave;  // same for every lane

        // U steps of R rows: lane takes chunk lane + 64*step.  A step past the
        // slice end re-reads the last chunk (in bounds) and is not used.
        auto load = [&](int s0, uint4 (&w)[U][R], uint16_t (&sb)[U][R], int16_t (&zb)[U][R]) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int cc = c0 + min(lane + (s0 + u) * kWave, nch - 1);
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    w[u][r] = packed[wrow[r] + cc];
                    sb[u][r] = scales[srow[r] + (cc >> gshift)];
                    zb[u][r] = ASYM ? zeros[srow[r] + (cc >> gshift)] : (int16_t)0;
                }
            }
        };
        auto compute = [&](int s0, const uint4 (&w)[U][R], const uint16_t (&sb)[U][R],
                           const int16_t (&zb)[U][R]) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = lane + (s0 + u) * kWave;
                if (c >= nch) break;
#pragma unroll
                for (int m = 0; m < MMAX; ++m) {
                    if (m >= M) break;
                    const uint4* xp = lds + m * (ks >> 3) + c * 4;
                    const uint4 x0 = xp[0], x1 = xp[1], x2 = xp[2], x3 = xp[3];
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        const float part = chunk_dot<ASYM>(w[u][r], x0, x1, x2, x3, zb[u][r], kc);
                        acc[m][r] = fmaf(f16_bits_to_f32(sb[u][r]), part, acc[m][r]);
                    }
                }
            }
        };

        uint4 wa[U][R], wb[U][R];
        uint16_t sa[U][R], sbb[U][R];
        int16_t za[U][R], zbb[U][R];
        // Weight loads go out before the activations are staged, so HBM is
        // busy while the block waits on its barrier.
        load(0, wa, sa, za);
        if (k0 > 0) __syncthreads();     // previous slice fully consumed
        stage_activations(X, M, K, k0, ks, lds, perm);
        __syncthreads();

        for (int s0 = 0; s0 < nsteps; s0 += 2 * U) {
            if (s0 + U < nsteps) load(s0 + U, wb, sbb, zbb);
            compute(s0, wa, sa, za);
            if (s0 + U >= nsteps) break;
            if (s0 + 2 * U < nsteps) load(s0 + 2 * U, wa, sa, za);
            compute(s0 + U, wb, sbb, zbb);
        }
    }

#pragma unroll
    for (int m = 0; m < MMAX; ++m) {
        if (m >= M) break;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float v = wave_sum_lane63(acc[m][r]);
            if (lane == kWave - 1 && row0 + r < N) Y[(size_t)m * N + row0 + r] = f32_to_f16_bits(v);
        }
    }
}

// Persistent variant for activations that fit LDS whole (M*K*2 bytes within
// the budget).  Each block stages X once; each wave then walks its row
// groups g, g + G, g + 2G, ... (G = waves in the grid) of R rows, and the
// (row group, chunk step) iterations form one stream with a ring of P
// prefetched steps, so loads for the next row group are in flight while the
// current one finishes and is reduced.
//   - Weights and scales come through raw buffer loads over the rows from
//     the group's first row to the end of the matrix: scalar addressing plus
//     one 32-bit lane offset, and reads past the last row return 0 without
//     touching memory.  Every load is issued unconditionally (steps past the
//     wave's work use an empty resource), so the compiler's counter waits are
//     exact and P steps really stay in flight.
//   - X is loaded into registers before the first weight loads, so staging
//     it waits only for its own loads.
//   - A lane whose chunk is past the end of the row (last partial step)
//     contributes with scale 0 and reads a valid LDS address.
//   - PERM (act order): X is staged unpaired with 16-byte loads, issued with
//     the matching 16-byte loads of perm (one memory round trip), and the
//     block then gathers x[perm[j]] from LDS (an index outside [0, K) reads
//     0) into the paired layout; the raw copy takes a second LDS region.
// XPT: 16-byte activation blocks staged per thread (MMAX*K/8 <= XPT*threads).
// LPR: lanes per row.  64: every lane of the wave works on the same R rows,
// lane l taking chunks l, l + 64, ...; 16: the wave holds four rows side by
// side per register slot (R * 4 rows a row group), lane l on row l / 16 and
// chunks l % 16, l % 16 + 16, ..., the sum over each 16-lane segment.  A row
// of K/32 chunks then fills whole steps when K/32 is a multiple of 16 but not
// of 64 (K = 3584: 7 steps of 16 lanes instead of 2 steps of 64 with 16 idle
// lanes in the second); chosen by gemv_lanes_per_row.
template <int MMAX, int R, int P, int WAVES, int XPT, bool ASYM, bool PERM, int LPR>
__global__ __launch_bounds__(WAVES * kWave) void gemv_persistent_kernel(
    const uint16_t* __restrict__ X, int M, const uint4* __restrict__ packed,
    const uint16_t* __restrict__ scales, const int16_t* __restrict__ zeros,
    uint16_t* __restrict__ Y, int N, int K, int gshift, const int* __restrict__ perm) {
    static_assert(LPR == kWave || LPR == 16, "lanes per row");
    constexpr int S = kWave / LPR;                         // rows side by side
    constexpr int RG = R * S;                              // rows per row group
    extern __shared__ uint4 lds[];
    const int lane = threadIdx.x & (kWave - 1);
    const int seg = lane / LPR, li = lane % LPR;           // row within a slot, lane in it
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int nchunks = K >> 5;
    if (nchunks == 0) return;  // K == 0 is launched on gemv_kernel, which writes the zeros
    const int nsteps = (nchunks + LPR - 1) / LPR;          // chunk steps per row group
    const int total_rg = (N + RG - 1) / RG;
    const int stride_rg = gridDim.x * WAVES;
    const int first_rg = blockIdx.x * WAVES + wave;
    const int my_rg = first_rg < total_rg ? (total_rg - 1 - first_rg) / stride_rg + 1 : 0;
    const int T = my_rg * nsteps;                          // this wave's iterations
    const uint32_t wrow_bytes = (uint32_t)K / 2;
    const uint32_t srow_bytes = (uint32_t)scales_per_row(K, gshift) * 2;  // one per 2^gshift chunks
    const CodeConsts kc = code_consts();

    // X blocks of this thread, loaded first (indices clamped into range).
    const int xblocks = M * (K >> 3);
    uint4 xr[XPT];
    int4 pr[PERM ? XPT : 1][2];
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
        const int e = min((int)threadIdx.x + i * WAVES * kWave, xblocks - 1);
        const int m = e / (K >> 3);
        const int col0 = (e - m * (K >> 3)) * 8;
        if constexpr (PERM) {
            xr[i] = x_block(X, m, K, col0, nullptr);          // unpermuted, contiguous
            pr[i][0] = reinterpret_cast<const int4*>(perm + col0)[0];
            pr[i][1] = reinterpret_cast<const int4*>(perm + col0)[1];
        } else {
            xr[i] = x_block(X, m, K, col0, perm);
        }
    }

    // load cursor (wave-uniform): iteration tl -> (row group lrg, step ls)
    int tl = 0, lrg = first_rg, ls = 0;
    __amdgpu_buffer_rsrc_t wr = buffer_rsrc(packed, 0), sr = buffer_rsrc(scales, 0);
    __amdgpu_buffer_rsrc_t zr = buffer_rsrc(zeros, 0);
    auto load = [&](uint4 (&wd)[R], uint16_t (&sd)[R], int16_t (&zd)[R]) {
        if (ls == 0) {
            // new row group (or past the wave's work: an empty resource)
            const bool live = tl < T;
            const int64_t row0 = (int64_t)lrg * RG;
            const int64_t rows_left = live ? (int64_t)N - row0 : 0;
            wr = buffer_rsrc(reinterpret_cast<const char*>(packed) + (live ? row0 * wrow_bytes : 0),
                             (uint64_t)rows_left * wrow_bytes);
            sr = buffer_rsrc(reinterpret_cast<const char*>(scales) + (live ? row0 * srow_bytes : 0),
                             (uint64_t)rows_left * srow_bytes);
            if constexpr (ASYM)
                zr = buffer_rsrc(reinterpret_cast<const char*>(zeros) + (live ? row0 * srow_bytes : 0),
                                 (uint64_t)rows_left * srow_bytes);
        }
        // row r * S + seg of the group: seg in the lane offset, r * S in the
        // scalar one (both count in the buffer's range check)
        const int voff_w = seg * (int)wrow_bytes + (li + ls * LPR) * 16;
        const int voff_s = seg * (int)srow_bytes + ((li + ls * LPR) >> gshift) * 2;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            typedef unsigned v4u __attribute__((ext_vector_type(4)));
            // streamed once: non-temporal (kStreamLoad) keeps them from
            // displacing reusable lines in L2
            const v4u v = __builtin_amdgcn_raw_buffer_load_b128(wr, voff_w, r * S * wrow_bytes,
                                                                 kStreamLoad);
            wd[r] = make_uint4(v.x, v.y, v.z, v.w);
            sd[r] = __builtin_amdgcn_raw_buffer_load_b16(sr, voff_s, r * S * srow_bytes,
                                                         kStreamLoad);
            zd[r] = ASYM ? (int16_t)__builtin_amdgcn_raw_buffer_load_b16(zr, voff_s,
                                                                         r * S * srow_bytes,
                                                                         kStreamLoad)
                         : (int16_t)0;
        }
        ++tl;
        if (++ls == nsteps) { ls = 0; lrg += stride_rg; }
    };

    // Ring of Q = P + 1 slots: iteration t computes slot t % Q after issuing
    // the load of iteration t + P into slot (t + P) % Q, the slot iteration
    // t - 1 consumed, so P steps stay in flight while a step is multiplied.
    constexpr int Q = P + 1;
    uint4 w[Q][R];
    uint16_t sb[Q][R];
    int16_t zb[Q][R];
#pragma unroll
    for (int i = 0; i < P; ++i) load(w[i], sb[i], zb[i]);

    if constexpr (PERM) {
        // raw X in the second region, then the gather through perm from LDS
        uint4* const raw = lds + xblocks;
#pragma unroll
        for (int i = 0; i < XPT; ++i) {
            const int e = (int)threadIdx.x + i * WAVES * kWave;
            if (e < xblocks) raw[e] = xr[i];
        }
        __syncthreads();
        const uint16_t* const rawh = reinterpret_cast<const uint16_t*>(raw);
#pragma unroll
        for (int i = 0; i < XPT; ++i) {
            const int e = (int)threadIdx.x + i * WAVES * kWave;
            if (e < xblocks) {
                const int m = e / (K >> 3);
                const int idx[8] = {pr[i][0].x, pr[i][0].y, pr[i][0].z, pr[i][0].w,
                                    pr[i][1].x, pr[i][1].y, pr[i][1].z, pr[i][1].w};
                uint32_t h[8];
#pragma unroll
                for (int b = 0; b < 8; ++b)
                    h[b] = (uint32_t)idx[b] < (uint32_t)K ? rawh[m * K + idx[b]] : 0u;
                lds[e] = pair_block(h[0] | (h[1] << 16), h[2] | (h[3] << 16),
                                    h[4] | (h[5] << 16), h[6] | (h[7] << 16));
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < XPT; ++i) {
            const int e = (int)threadIdx.x + i * WAVES * kWave;
            if (e < xblocks) lds[e] = pair_block(xr[i].x, xr[i].y, xr[i].z, xr[i].w);
        }
    }
    __syncthreads();

    int crg = first_rg;   // compute cursor (wave-uniform)
    int cs = 0;
    float acc[MMAX][R];
#pragma unroll
    for (int m = 0; m < MMAX; ++m)
#pragma unroll
        for (int r = 0; r < R; ++r) acc[m][r] = 0.0f;

    for (int t0 = 0; t0 < T; t0 += Q) {
#pragma unroll
        for (int i = 0; i < Q; ++i) {
            load(w[(i + P) % Q], sb[(i + P) % Q], zb[(i + P) % Q]);   // iteration t0 + i + P
            const int c = li + cs * LPR;
            const bool valid = c < nchunks;
            const int cx = min(c, nchunks - 1);
            // Steps past the wave's work (the ring's tail) skip the arithmetic;
            // the branch is wave-uniform and holds no loads.
#pragma unroll
            for (int m = 0; m < MMAX; ++m) {
                if (m >= M || t0 + i >= T) break;
                const uint4* xp = lds + m * (K >> 3) + cx * 4;
                const uint4 x0 = xp[0], x1 = xp[1], x2 = xp[2], x3 = xp[3];
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const float part = chunk_dot<ASYM>(w[i][r], x0, x1, x2, x3, zb[i][r], kc);
                    const float sc = valid ? f16_bits_to_f32(sb[i][r]) : 0.0f;
                    acc[m][r] = fmaf(sc, part, acc[m][r]);
                }
            }
            if (++cs == nsteps) {
                cs = 0;
                if (t0 + i < T) {
                    // row group complete: reduce over the wave and store
#pragma unroll
                    for (int m = 0; m < MMAX; ++m) {
                        if (m >= M) break;
#pragma unroll
                        for (int r = 0; r < R; ++r) {
                            const float v = LPR == kWave ? wave_sum_lane63(acc[m][r])
                                                         : row16_sum(acc[m][r]);
                            const int row = crg * RG + r * S + seg;
                            if (li == LPR - 1 && row < N)
                                Y[(size_t)m * N + row] = f32_to_f16_bits(v);
                            acc[m][r] = 0.0f;
                        }
                    }
                }
                crg += stride_rg;
            }
        }
    }
}

namespace {

constexpr int kLdsBudget = 64 * 1024;

template <int MMAX, int R, int U, int WAVES, bool ASYM>
hipError_t launch_gemv_t(const uint16_t* X, int64_t M, const uint32_t* packed,
                         const uint16_t* scales, const int16_t* zeros, int64_t N, int64_t K,
                         uint16_t* Y, hipStream_t stream, int gshift, const int* perm) {
    // LDS: 2 bytes per activation element.
    int64_t kslice = (int64_t)(kLdsBudget / (MMAX * 2)) / kGroup * kGroup;
    if (kslice > K) kslice = K;
    if (kslice < kGroup) kslice = kGroup;
    const size_t lds = (size_t)MMAX * (kslice / 8) * sizeof(uint4);
    const int64_t rows_per_block = (int64_t)R * WAVES;
    const int64_t blocks = (N + rows_per_block - 1) / rows_per_block;
    hipLaunchKernelGGL((gemv_kernel<MMAX, R, U, WAVES, ASYM>), dim3((unsigned)blocks),
                       dim3(WAVES * kWave), lds, stream, X, (int)M,
                       reinterpret_cast<const uint4*>(packed), scales, zeros, Y, (int)N, (int)K,
                       (int)kslice, gshift, perm);
    return hipGetLastError();
}

// Grid: a whole number b of blocks per compute unit, b at most
// blocks_per_cu and at most what one compute unit holds at once (the
// runtime's occupancy for this kernel and LDS size), so that with
// grid-stride row groups every compute unit gets the same work to within
// one row group per wave and no block waits for a second round.  Measured
// on gfx950, M = 1: 4096x28672 12.4-12.5 us with 2048 blocks against
// 13.8-14.2 us with 1195 (4.67 blocks per CU leave the CUs with a fifth
// block 7 % more work), 4096x14336 7.5-7.8 us against 8.6-8.9 us with 896.
// Fewer row groups than waves on the chip: one wave per row group.
template <int MMAX, int R, int P, int WAVES, int XPT, bool ASYM, bool PERM, int LPR>
hipError_t launch_persistent_kern(const uint16_t* X, int64_t M, const uint32_t* packed,
                                  const uint16_t* scales, const int16_t* zeros, int64_t N,
                                  int64_t K, uint16_t* Y, hipStream_t stream, int num_cu,
                                  int blocks_per_cu, int gshift, const int* perm);

template <int MMAX, int R, int P, int WAVES, int XPT, bool ASYM>
hipError_t launch_persistent_xpt(const uint16_t* X, int64_t M, const uint32_t* packed,
                                 const uint16_t* scales, const int16_t* zeros, int64_t N,
                                 int64_t K, uint16_t* Y, hipStream_t stream, int num_cu,
                                 int blocks_per_cu, int gshift, const int* perm) {
#define W4A16_PERSISTENT_KERN(PERM, LPR)                                                     \
    launch_persistent_kern<MMAX, R, P, WAVES, XPT, ASYM, PERM, LPR>(                         \
        X, M, packed, scales, zeros, N, K, Y, stream, num_cu, blocks_per_cu, gshift, perm)
    if constexpr (MMAX == 1) {
        if (gemv_lanes_per_row(K, N, num_cu) == 16)
            return perm != nullptr ? W4A16_PERSISTENT_KERN(true, 16)
                                   : W4A16_PERSISTENT_KERN(false, 16);
    }
    return perm != nullptr ? W4A16_PERSISTENT_KERN(true, kWave) : W4A16_PERSISTENT_KERN(false, kWave);
#undef W4A16_PERSISTENT_KERN
}

template <int MMAX, int R, int P, int WAVES, int XPT, bool ASYM, bool PERM, int LPR>
hipError_t launch_persistent_kern(const uint16_t* X, int64_t M, const uint32_t* packed,
                                  const uint16_t* scales, const int16_t* zeros, int64_t N,
                                  int64_t K, uint16_t* Y, hipStream_t stream, int num_cu,
                                  int blocks_per_cu, int gshift, const int* perm) {
    // paired X; with perm also the raw copy it is gathered from
    const size_t lds = (size_t)(PERM ? 2 : 1) * MMAX * (K / 8) * sizeof(uint4);
    auto kern = gemv_persistent_kernel<MMAX, R, P, WAVES, XPT, ASYM, PERM, LPR>;
    if (lds > 64 * 1024) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 (int)lds);
        if (e != hipSuccess) return e;
    }
    // resident blocks per CU for the last LDS size seen (lds << 8 | blocks)
    static std::atomic<uint64_t> occ_cache{0};
    uint64_t c = occ_cache.load(std::memory_order_relaxed);
    int resident = (int)(c & 0xFF);
    if ((c >> 8) != (uint64_t)lds || resident == 0) {
        int nb = 0;
        const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &nb, reinterpret_cast<const void*>(kern), WAVES * kWave, lds);
        if (e != hipSuccess) return e;
        resident = nb < 1 ? 1 : (nb > 255 ? 255 : nb);
        occ_cache.store(((uint64_t)lds << 8) | (uint64_t)resident, std::memory_order_relaxed);
    }
    constexpr int64_t RG = (int64_t)R * (kWave / LPR);        // rows per row group
    const int64_t total_rg = (N + RG - 1) / RG;
    const int64_t per_cu = (int64_t)num_cu * WAVES;
    int64_t blocks = (total_rg + WAVES - 1) / WAVES;
    if (total_rg >= per_cu) {
        int64_t b = total_rg / per_cu;
        if (b > blocks_per_cu) b = blocks_per_cu;
        if (b > resident) b = resident;
        blocks = b * num_cu;
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(WAVES * kWave), lds, stream, X, (int)M,
                       reinterpret_cast<const uint4*>(packed), scales, zeros, Y, (int)N, (int)K,
                       gshift, perm);
    return hipGetLastError();
}

template <int MMAX, int R, int P, int WAVES, bool ASYM>
hipError_t launch_persistent_t(const uint16_t* X, int64_t M, const uint32_t* packed,
                               const uint16_t* scales, const int16_t* zeros, int64_t N,
                               int64_t K, uint16_t* Y, hipStream_t stream, int num_cu,
                               int blocks_per_cu, int gshift, const int* perm) {
    const int64_t need = (int64_t)MMAX * (K / 8);             // x blocks to stage
    const int64_t threads = (int64_t)WAVES * kWave;
#define W4A16_PERSISTENT(XPT)                                                                  \
    launch_persistent_xpt<MMAX, R, P, WAVES, XPT, ASYM>(X, M, packed, scales, zeros, N, K, Y,  \
                                                        stream, num_cu, blocks_per_cu, gshift, \
                                                        perm)
    if (need <= threads) return W4A16_PERSISTENT(1);
    if (need <= 2 * threads) return W4A16_PERSISTENT(2);
    if (need <= 4 * threads) return W4A16_PERSISTENT(4);
    if (need <= 8 * threads) return W4A16_PERSISTENT(8);
    return W4A16_PERSISTENT(16);
#undef W4A16_PERSISTENT
}

// Launch choice (measured on MI355X over the decode layer shapes, K x N from
// 4096x1024 to 8192x28672, with the (P+1)-slot ring and non-temporal loads):
// whole-X staging with the persistent kernel when it fits; two rows per
// wave; for K up to 8192 one step in flight, four waves per block, up to
// eight blocks per compute unit; for longer rows (K >= 12288, where the
// per-block activation copy is larger) eight waves per block, up to two
// blocks per compute unit.
template <int MMAX, bool ASYM>
hipError_t launch_gemv_m(const uint16_t* X, int64_t M, const uint32_t* packed,
                         const uint16_t* scales, const int16_t* zeros, int64_t N, int64_t K,
                         uint16_t* Y, hipStream_t stream, int num_cu, int gshift,
                         const int* perm) {
    if (K > 0 && (int64_t)MMAX * K * 2 <= kLdsBudget) {
        constexpr int R = MMAX >= 4 ? 1 : 2;
        // Measured on gfx950 for M = 1: long rows (K = 14336) run best with
        // 8 waves per block, 2 blocks per CU and one step in flight (7.9 us
        // against 8.6 us with two steps in flight).
        if (MMAX == 1 && K >= 12288)
            return launch_persistent_t<1, 2, 1, 8, ASYM>(X, M, packed, scales, zeros, N, K, Y,
                                                         stream, num_cu, 2, gshift, perm);
        if (K >= 12288)
            return launch_persistent_t<MMAX, R, 2, 8, ASYM>(X, M, packed, scales, zeros, N, K, Y,
                                                            stream, num_cu, 2, gshift, perm);
        // Every block gathers its own copy of x through perm, so act-order
        // launches use fewer blocks (4096x14336: 15.3 us with 8 per CU).
        return launch_persistent_t<MMAX, R, 1, 4, ASYM>(X, M, packed, scales, zeros, N, K, Y,
                                                        stream, num_cu, perm ? 4 : 8, gshift,
                                                        perm);
    }
    constexpr int WAVES = 4;
    if constexpr (MMAX <= 4) {
        // four rows per wave only for up to four rows of X (more would not
        // fit the register file)
        if (N >= (int64_t)4 * WAVES * num_cu)
            return launch_gemv_t<MMAX, 4, 2, WAVES, ASYM>(X, M, packed, scales, zeros, N, K, Y,
                                                          stream, gshift, perm);
    }
    if (N >= (int64_t)2 * WAVES * num_cu)
        return launch_gemv_t<MMAX, 2, 2, WAVES, ASYM>(X, M, packed, scales, zeros, N, K, Y,
                                                      stream, gshift, perm);
    return launch_gemv_t<MMAX, 1, 4, WAVES, ASYM>(X, M, packed, scales, zeros, N, K, Y, stream,
                                                  gshift, perm);
}

template <bool ASYM>
hipError_t launch_gemv_a(const uint16_t* X, int64_t M, const uint32_t* packed,
                         const uint16_t* scales, const int16_t* zeros, int64_t N, int64_t K,
                         uint16_t* Y, hipStream_t stream, int num_cu, int gshift,
                         const int* perm) {
    if (M == 1)
        return launch_gemv_m<1, ASYM>(X, M, packed, scales, zeros, N, K, Y, stream, num_cu,
                                      gshift, perm);
    if (M == 2)
        return launch_gemv_m<2, ASYM>(X, M, packed, scales, zeros, N, K, Y, stream, num_cu,
                                      gshift, perm);
    if (M <= 4)
        return launch_gemv_m<4, ASYM>(X, M, packed, scales, zeros, N, K, Y, stream, num_cu,
                                      gshift, perm);
    // M > 8 is split into slices of at most 8 activation rows.
    for (int64_t m0 = 0; m0 < M; m0 += 8) {
        const int64_t mm = (M - m0 < 8) ? (M - m0) : 8;
        hipError_t e = launch_gemv_m<8, ASYM>(X + m0 * K, mm, packed, scales, zeros, N, K,
                                              Y + m0 * N, stream, num_cu, gshift, perm);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_gemv_valu(const uint16_t* X, int64_t M, const uint32_t* packed,
                            const uint16_t* scales, int64_t N, int64_t K, uint16_t* Y,
                            hipStream_t stream, int num_cu, int gshift, const int* perm,
                            const int16_t* zeros) {
    if (zeros != nullptr)
        return launch_gemv_a<true>(X, M, packed, scales, zeros, N, K, Y, stream, num_cu, gshift,
                                   perm);
    return launch_gemv_a<false>(X, M, packed, scales, nullptr, N, K, Y, stream, num_cu, gshift,
                                perm);
}

}  // namespace w4a16

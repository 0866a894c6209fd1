// gemm_mfma.hip — W4A16 GEMM on the gfx950 matrix cores (batched decode,
// M >= 16, and prefill, [BENCH] §一 512-token prompt, §二 prefill latency).
//
// Y[m,n] = sum_k X[m,k] * fp16(s[n,k/group] * q[n,k]), fp32 accumulation in
// v_mfma_f32_16x16x32_f16, fp16 output.  group: 32, 64, 128, 256 or the
// whole row ([QUANT] sub-section 3, granularity), passed as gshift =
// log2(group / 32); the kernel walks K in steps of 128 either way.
//
// Operand mapping of v_mfma_f32_16x16x32_f16 (lane l, j = l/16):
//   A (16 x 32): row l%16, eight k values of slot j
//   B (32 x 16): column l%16, eight k values of slot j
//   D (16 x 16): rows 4j..4j+3 of column l%16
// The contraction does not depend on which k a slot holds as long as A and
// B agree, so a lane's B operand for the four k-steps of a 128-wide group is
// one 16-byte load of its row: words 4j..4j+3 (elements 32j .. 32j+31), word
// 4j+kk feeding k-step kk.  The word is dequantized in registers to
// fp16(s*q) in the paired order of dequant_word(), and A is staged in LDS in
// the same paired order (pair_block), so no B tile passes through LDS.
//
// Block: WM x WN x WK waves.  A wave computes a (16 TM) x (16 TN) tile;
// WK > 1 splits the groups of K over waves (for few output tiles) and the
// partial tiles are summed through LDS at the end.  Every load offset is a
// per-thread 32-bit offset from the block's first row, fixed for the whole
// K loop (rows past M or N clamped to the last row), so the loop has no
// masking; X is double-buffered in LDS (one barrier per K step) and the B
// registers of two steps alternate.  The prefill tiles (SST) stage each
// step's scales (and zero points) through LDS beside its X tile: one 2-byte
// load per column for the whole block instead of one per lane and wave.
// Precision: fp16(s*q) has relative error <= 2^-11, so |y - y_exact| <=
// 2^-11 sum |x w| plus fp32 accumulation error, inside the 1e-3 sum |x w|
// allowance for every K.  The block scans its scales once: a group with
// absmax 65504 (s = 9360, 7 s rounds to infinity in fp16) sends the block to
// a second copy of the K loop that clamps its fp16 weights to +-65504.
//
// Asymmetric weights (ASYM, [QUANT] sub-section 2: w = s (n - z), nibble n
// in [0, 15], an integer zero point z per group): where the block's scales
// are all below 64 and its zero points within +-1000, B holds fp16(s (n - z))
// formed from the exact codes n - z (codes_word_zp), multiplied as the
// symmetric weights are.  Otherwise (s (n - z) may leave the fp16 range) the
// block runs an exact copy of the loop: B holds the codes n - zc (zc = z
// clamped to +-1000), each group's MFMA sums are scaled once in fp32, and a
// group with |z| > 1000 adds s (zc - z) times the group's activation sums,
// which an MFMA against a B of ones forms in the same pass.
#include "w4a16_device.h"
#include "w4a16_launch.h"
#include "w4a16_fp16_weights.h"

namespace w4a16 {

namespace {
constexpr int kLdaHalfs = 136;             // staged A row: 128 halves + 8 pad (bank spread)
constexpr int kLdaVec = kLdaHalfs / 8;     // in uint4
constexpr int kCoherentSc1 = 16;           // cache policy: coherent at device scope (sc1)
}  // namespace

// PART: 0 = both copies of the K loop (the block picks one); 1 = the common
// copy only (a block that needs the slow copy returns at once); 2 = the slow
// copy only, deciding over the scale_bn columns around the block (the block
// tile of the PART 1 launch it completes), so that the two launches split
// the blocks between them exactly.
template <int TM, int TN, int WM, int WN, int WK, bool ASYM, bool SPLIT, int PART, bool SST>
__global__ __launch_bounds__(WM * WN * WK * kWave)
__attribute__((amdgpu_waves_per_eu(2))) void gemm_mfma_kernel(
    const uint16_t* __restrict__ X, int M, const uint4* __restrict__ packed,
    const uint16_t* __restrict__ scales, const int16_t* __restrict__ zeros,
    uint16_t* __restrict__ Y, int N, int K, int gshift, int ksplit, int gps,
    float4_t* __restrict__ partials, int scan_bn) {
    static_assert(!SPLIT || WK == 1, "the K split sums whole block tiles");
    static_assert(!SPLIT || PART == 0, "the K split runs both copies");
    constexpr int NT = WM * WN * WK * kWave;
    constexpr int BM = 16 * TM * WM;
    constexpr int BN = 16 * TN * WN;
    constexpr int A_VECS = WK * BM * 16;              // uint4 of A per stage (WK groups)
    constexpr int A_PER_THREAD = A_VECS / NT;
    static_assert(A_VECS % NT == 0, "A staging must tile the block");
    // Stage vector v = i NT + thread is (group slot v / (16 BM), row, 8-block);
    // when a slot spans whole passes of the block, vector i's slot is the
    // same for every thread.
    constexpr bool SLOT_UNIFORM = (BM * 16) % NT == 0;
    constexpr int LDS_STAGE = WK * BM * kLdaVec;      // uint4 per A buffer
    extern __shared__ uint4 lds[];                    // [2][WK][BM][kLdaVec], then (SST)
                                                      // [2][kinds][WK][BN] scales, zero points
    // SST (one scale per step or fewer, group >= 128): the scales (and zero
    // points) of a step are staged through LDS beside its A tile, one 2-byte
    // load per column and group slot for the whole block, instead of one per
    // lane, row and step (the lanes of a column would otherwise issue the
    // same scattered 2-byte loads from every wave).
    constexpr int KINDS = ASYM ? 2 : 1;
    constexpr int SCOLS = WK * BN;                    // scales per step and block
    constexpr int S_PER_THREAD = SST ? (KINDS * SCOLS + NT - 1) / NT : 1;
    static_assert(!SST || BN % kWave == 0, "a wave stages one kind and group slot");

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int wk = wave % WK;
    const int wn = (wave / WK) % WN;
    const int wm = wave / (WK * WN);
    const int l16 = lane & 15;
    const int j = lane >> 4;
    const int m_blk = blockIdx.y * BM;
    const int n_blk = blockIdx.x * BN;
    // K split over blocks (SPLIT): block z of a tile takes the groups
    // [z gps, z gps + gps) of K (every slice holds at least one).
    const int g_lo = SPLIT ? (int)blockIdx.z * gps : 0;
    const int ngroups = SPLIT ? min(K >> 7, g_lo + gps) - g_lo : (K >> 7);   // 128-element steps
    const int nsteps = (ngroups + WK - 1) / WK;
    const uint32_t wrow = (uint32_t)K / 2;            // bytes per weight row
    // bytes per scale (and zero) row: one scale per 2^gshift chunks of 32
    const uint32_t srow = (uint32_t)scales_per_row(K, gshift) * 2;
    // Lane j's 32 elements of a 128-element step are chunk 4 g + j of its row,
    // whose scale is number (4 g + j) >> gshift: below group 128 the lane's
    // share (j >> gshift) is fixed here and the step adds g << (2 - gshift);
    // from group 128 up every lane of the step reads scale g >> (gshift - 2)
    // (0 for one scale per row).
    const uint32_t s_lane = gshift < 2 ? (uint32_t)(j >> gshift) * 2u : 0u;

    // Byte offsets of this thread's loads from the block's first row, fixed
    // for the whole K loop (32-bit: the launcher keeps BM rows of X and BN
    // rows of codes below 2^31 bytes).  Rows past M or N are clamped to the
    // last row: they only feed outputs that are never stored.
    uint32_t a_off[A_PER_THREAD], a_lds[A_PER_THREAD];
    int a_slot[A_PER_THREAD];
#pragma unroll
    for (int i = 0; i < A_PER_THREAD; ++i) {
        constexpr int per_slot = SLOT_UNIFORM ? (BM * 16) / NT : 1;   // vectors i per slot
        const int v = i * NT + (int)threadIdx.x;
        const int slot = SLOT_UNIFORM ? i / per_slot : v / (BM * 16);
        const int rem = SLOT_UNIFORM ? (i % per_slot) * NT + (int)threadIdx.x : v % (BM * 16);
        const int row = rem >> 4;
        const int blk = rem & 15;
        const uint32_t m = (uint32_t)(min(m_blk + row, M - 1) - m_blk);
        a_off[i] = m * (uint32_t)K * 2u + (uint32_t)(slot * 256 + blk * 16);
        a_lds[i] = (uint32_t)((slot * BM + row) * kLdaVec + blk);
        a_slot[i] = slot;
    }
    uint32_t b_off[TN], s_off[TN];
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
        const uint32_t r = (uint32_t)(min(n_blk + (wn * TN + tn) * 16 + l16, N - 1) - n_blk);
        b_off[tn] = r * wrow + (uint32_t)j * 16u;
        s_off[tn] = r * srow + s_lane;
    }
    // Buffer resources over the block's rows; loads take the per-thread
    // offset in a VGPR and the step's offset in an SGPR.
    typedef unsigned v4u __attribute__((ext_vector_type(4)));
    const __amdgpu_buffer_rsrc_t xr = buffer_rsrc(
        reinterpret_cast<const char*>(X) + (size_t)m_blk * K * 2, (uint64_t)(M - m_blk) * K * 2);
    const __amdgpu_buffer_rsrc_t pr = buffer_rsrc(
        reinterpret_cast<const char*>(packed) + (size_t)n_blk * wrow, (uint64_t)(N - n_blk) * wrow);
    const __amdgpu_buffer_rsrc_t sr = buffer_rsrc(
        reinterpret_cast<const char*>(scales) + (size_t)n_blk * srow, (uint64_t)(N - n_blk) * srow);
    const __amdgpu_buffer_rsrc_t zr =
        ASYM ? buffer_rsrc(reinterpret_cast<const char*>(zeros) + (size_t)n_blk * srow,
                           (uint64_t)(N - n_blk) * srow)
             : sr;

    // Scale staging entries of this thread (SST): entry e = thread + i NT is
    // (kind, group slot, column); a wave's entries are of one kind.
    uint16_t* const slds = reinterpret_cast<uint16_t*>(lds + 2 * LDS_STAGE);
    uint32_t st_row[S_PER_THREAD];
    int st_slot[S_PER_THREAD], st_idx[S_PER_THREAD];
    bool st_zero[S_PER_THREAD], st_live[S_PER_THREAD];
#pragma unroll
    for (int i = 0; i < S_PER_THREAD; ++i) {
        // kind, slot and liveness from the wave's first entry (BN is a
        // multiple of the wave, so they are the same for all its lanes)
        const int e_wave = __builtin_amdgcn_readfirstlane(((int)threadIdx.x & ~(kWave - 1)) + i * NT);
        const int col = ((int)threadIdx.x + i * NT) % BN;
        st_live[i] = e_wave < KINDS * SCOLS;
        st_zero[i] = e_wave >= SCOLS;
        st_slot[i] = (e_wave % SCOLS) / BN;
        st_row[i] = (uint32_t)(min(n_blk + col, N - 1) - n_blk) * srow;
        st_idx[i] = ((st_zero[i] ? 1 : 0) * WK + st_slot[i]) * BN + col;
    }
    // Entries past the last group read 0 through an empty resource (scale 0,
    // zero point 0: such a group's codes are 8 and its A slot stale, so its
    // product must vanish).
    const __amdgpu_buffer_rsrc_t s_empty = buffer_rsrc(scales, 0);
    uint32_t s_regs[S_PER_THREAD];
    auto load_s = [&](int step) {
        if constexpr (SST) {
#pragma unroll
            for (int i = 0; i < S_PER_THREAD; ++i) {
                const int g = step * WK + st_slot[i];
                const int sg = (g_lo + g) >> (gshift - 2);
                const bool live = st_live[i] && g < ngroups;      // wave-uniform
                s_regs[i] = __builtin_amdgcn_raw_buffer_load_b16(
                    live ? (st_zero[i] ? zr : sr) : s_empty, st_row[i] + (uint32_t)sg * 2u, 0, 0);
            }
        }
    };
    auto store_s = [&](int buf) {
        if constexpr (SST) {
#pragma unroll
            for (int i = 0; i < S_PER_THREAD; ++i)
                if (st_live[i]) slds[buf * KINDS * SCOLS + st_idx[i]] = (uint16_t)s_regs[i];
        }
    };

    // A staging: vector i of the stage is (group slot, row, 8-block).  A
    // slot past the last group keeps its previous (finite) values; the B of
    // such a group is zero.
    auto load_a = [&](int step, uint4 (&regs)[A_PER_THREAD]) {
        const int soff = (g_lo + step * WK) * 256;
#pragma unroll
        for (int i = 0; i < A_PER_THREAD; ++i)
            if (step * WK + a_slot[i] < ngroups) {
                const v4u v = __builtin_amdgcn_raw_buffer_load_b128(xr, a_off[i], soff, 0);
                regs[i] = make_uint4(v.x, v.y, v.z, v.w);
            }
    };
    auto store_a = [&](int buf, const uint4 (&regs)[A_PER_THREAD]) {
        uint4* dst = lds + buf * LDS_STAGE;
#pragma unroll
        for (int i = 0; i < A_PER_THREAD; ++i)
            dst[a_lds[i]] = pair_block(regs[i].x, regs[i].y, regs[i].z, regs[i].w);
    };
    struct BRegs {
        uint4 w[TN];
        uint32_t s[TN];
        int z[TN];
    };
    auto load_b = [&](int step, BRegs& b) {
        const int g = step * WK + wk;
        if (g < ngroups) {
            const int ga = g_lo + g;                     // group index along the whole row
            const int sg = gshift <= 2 ? ga << (2 - gshift) : ga >> (gshift - 2);
#pragma unroll
            for (int tn = 0; tn < TN; ++tn) {
                const v4u v = __builtin_amdgcn_raw_buffer_load_b128(pr, b_off[tn], ga * 64, 0);
                b.w[tn] = make_uint4(v.x, v.y, v.z, v.w);
                if constexpr (SST) {
                    b.s[tn] = 0;                         // read from LDS in the step
                    b.z[tn] = 0;
                } else {
                    b.s[tn] = __builtin_amdgcn_raw_buffer_load_b16(sr, s_off[tn], sg * 2, 0);
                    b.z[tn] = ASYM ? (int)(int16_t)__builtin_amdgcn_raw_buffer_load_b16(
                                         zr, s_off[tn], sg * 2, 0)
                                   : 0;
                }
            }
        } else {
#pragma unroll
            for (int tn = 0; tn < TN; ++tn) {
                b.w[tn] = make_uint4(0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u);
                b.s[tn] = 0;
                b.z[tn] = 0;
            }
        }
    };

    const CodeConsts kc = code_consts();
    float4_t acc[TM][TN];
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) acc[tm][tn] = (float4_t){0.f, 0.f, 0.f, 0.f};

    // One step: multiply the group(s) of step s (A in LDS buffer s & 1, B in
    // cur), then store the A of step s + 1 (in registers since step s - 1)
    // to the other buffer and load A and B of step s + 2.  One barrier per
    // step orders both buffers.
    uint4 a_regs[A_PER_THREAD];
#pragma unroll
    for (int i = 0; i < A_PER_THREAD; ++i) a_regs[i] = make_uint4(0, 0, 0, 0);
    BRegs b0, b1;
    auto step_body = [&](int step, BRegs& cur, auto clamp) __attribute__((always_inline)) {
        const uint4* abase =
            lds + (step & 1) * LDS_STAGE + (wk * BM + wm * TM * 16 + l16) * kLdaVec + 4 * j;
        if constexpr (SST) {
            const uint16_t* sb = slds + (step & 1) * KINDS * SCOLS + wk * BN + wn * TN * 16 + l16;
#pragma unroll
            for (int tn = 0; tn < TN; ++tn) {
                cur.s[tn] = sb[tn * 16];
                if constexpr (ASYM) cur.z[tn] = (int)(int16_t)sb[WK * BN + tn * 16];
            }
        }
        if constexpr (ASYM) {
            // Common blocks (every scale below 64, every |z| <= 1000): fp16
            // weights s * (n - z) from the exact codes n - z, |s (n - z)| <
            // 64 * 1015 stays in the fp16 range; multiplied as the symmetric
            // weights are.  The slow copy keeps the codes exact and scales
            // each group's MFMA sums in fp32 (ŵ itself may exceed the fp16
            // range there), over half of the wave's row tiles at a time to
            // bound the temporaries; a group with |z| > 1000 adds s (zc - z)
            // times the group's activation sums (an MFMA against ones).
            auto mma = [&](auto slow) __attribute__((always_inline)) {
                if constexpr (!decltype(slow)::value) {
                    half8_t bf[TN][4];
#pragma unroll
                    for (int tn = 0; tn < TN; ++tn) {
                        const ZeroBias zb = zero_bias(cur.z[tn]);
                        const _Float16 sh = __builtin_bit_cast(_Float16, (uint16_t)cur.s[tn]);
                        const half2_t s2 = {sh, sh};
                        const uint32_t words[4] = {cur.w[tn].x, cur.w[tn].y, cur.w[tn].z,
                                                   cur.w[tn].w};
#pragma unroll
                        for (int kk = 0; kk < 4; ++kk) {
                            half2_t q[4];
                            codes_word_zp(words[kk], kc, zb, q);
                            const half2_t h0 = q[0] * s2, h1 = q[1] * s2, h2 = q[2] * s2,
                                          h3 = q[3] * s2;
                            bf[tn][kk] = (half8_t){h0.x, h0.y, h1.x, h1.y,
                                                   h2.x, h2.y, h3.x, h3.y};
                        }
                    }
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
                        for (int tm = 0; tm < TM; ++tm) {
                            const half8_t af =
                                __builtin_bit_cast(half8_t, abase[tm * 16 * kLdaVec + kk]);
#pragma unroll
                            for (int tn = 0; tn < TN; ++tn)
                                acc[tm][tn] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                                    af, bf[tn][kk], acc[tm][tn], 0, 0, 0);
                        }
                    }
                } else if (gshift >= 2) {
                    half8_t bq[TN][4];
                    float sf[TN], cf[TN];
#pragma unroll
                    for (int tn = 0; tn < TN; ++tn) {
                        const ZeroBias zb = zero_bias(cur.z[tn]);
                        sf[tn] = f16_bits_to_f32((uint16_t)cur.s[tn]);
                        cf[tn] = sf[tn] * (float)(zb.zc - cur.z[tn]);   // 0 for |z| <= 1000
                        const uint32_t words[4] = {cur.w[tn].x, cur.w[tn].y, cur.w[tn].z,
                                                   cur.w[tn].w};
#pragma unroll
                        for (int kk = 0; kk < 4; ++kk) {
                            half2_t q[4];
                            codes_word_zp(words[kk], kc, zb, q);
                            bq[tn][kk] = (half8_t){q[0].x, q[0].y, q[1].x, q[1].y,
                                                   q[2].x, q[2].y, q[3].x, q[3].y};
                        }
                    }
                    constexpr int TH = TM > 1 ? TM / 2 : 1;
                    const _Float16 one = (_Float16)1.0f;
                    const half8_t ones = {one, one, one, one, one, one, one, one};
                    // The activation sums are formed in every wave, also where
                    // no zero point exceeds +-1000 (cf = 0 there): an MFMA
                    // skipped by a branch would leave the MFMA results read
                    // below fewer wait states after it than the matrix core
                    // needs on the path that skips it.
#pragma unroll
                    for (int t0 = 0; t0 < TM; t0 += TH) {
                        // d: the group's products per row tile; xs: its
                        // activation sums
                        float4_t d[TH][TN], xs[TH];
#pragma unroll
                        for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
                            for (int th = 0; th < TH; ++th) {
                                const half8_t af = __builtin_bit_cast(
                                    half8_t, abase[(t0 + th) * 16 * kLdaVec + kk]);
#pragma unroll
                                for (int tn = 0; tn < TN; ++tn)
                                    d[th][tn] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                                        af, bq[tn][kk],
                                        kk == 0 ? (float4_t){0.f, 0.f, 0.f, 0.f} : d[th][tn], 0,
                                        0, 0);
                                xs[th] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                                    af, ones, kk == 0 ? (float4_t){0.f, 0.f, 0.f, 0.f} : xs[th],
                                    0, 0, 0);
                            }
                        }
#pragma unroll
                        for (int th = 0; th < TH; ++th)
#pragma unroll
                            for (int tn = 0; tn < TN; ++tn)
#pragma unroll
                                for (int r = 0; r < 4; ++r)
                                    acc[t0 + th][tn][r] =
                                        fmaf(cf[tn], xs[th][r],
                                             fmaf(sf[tn], d[th][tn][r], acc[t0 + th][tn][r]));
                    }
                } else {
                    // Groups of 32 or 64: the four 32-element chunks of a
                    // step have their own scales, and one MFMA of the common
                    // mapping sums over the chunks of the lanes j = 0..3.  Here
                    // the mapping is transposed: MFMA kk takes chunk kk, its
                    // slot j the vector 4 kk + j of the staged A row and word
                    // 4 kk + j of the weight row, which lane (l16, kk) loaded
                    // as its word j; so every MFMA (two for group 64) sums one
                    // group, scaled once in fp32 with the scale and zero point
                    // that lane (l16, kk) loaded.
                    const uint4* abase_t = abase - 3 * j;      // vector j of the row
                    half8_t bq[TN][4];
                    float sk[TN][4], ck[TN][4];
#pragma unroll
                    for (int tn = 0; tn < TN; ++tn) {
                        const ZeroBias zown = zero_bias(cur.z[tn]);
                        const float sown = f16_bits_to_f32((uint16_t)cur.s[tn]);
                        const float cown = sown * (float)(zown.zc - cur.z[tn]);
                        const uint32_t words[4] = {cur.w[tn].x, cur.w[tn].y, cur.w[tn].z,
                                                   cur.w[tn].w};
#pragma unroll
                        for (int kk = 0; kk < 4; ++kk) {
                            const int src = l16 + 16 * kk;
                            // word 4 kk + j: word j of lane (l16, kk)
                            uint32_t wt = 0;
#pragma unroll
                            for (int r = 0; r < 4; ++r) {
                                const uint32_t v = (uint32_t)__shfl((int)words[r], src);
                                wt = r == j ? v : wt;
                            }
                            sk[tn][kk] = __shfl(sown, src);
                            ck[tn][kk] = __shfl(cown, src);
                            half2_t q[4];
                            codes_word_zp(wt, kc, zero_bias(__shfl(cur.z[tn], src)), q);
                            bq[tn][kk] = (half8_t){q[0].x, q[0].y, q[1].x, q[1].y,
                                                   q[2].x, q[2].y, q[3].x, q[3].y};
                        }
                    }
                    const _Float16 one = (_Float16)1.0f;
                    const half8_t ones = {one, one, one, one, one, one, one, one};
                    // LAST: chunks per group - 1 (0 for group 32, 1 for 64), a
                    // constant in each copy so that no branch separates an
                    // MFMA from the fold that reads it (as above).
                    auto groups = [&](auto last_c) __attribute__((always_inline)) {
                        constexpr int LAST = decltype(last_c)::value;
#pragma unroll
                        for (int tm = 0; tm < TM; ++tm) {
                            float4_t d[TN], xs;
#pragma unroll
                            for (int kk = 0; kk < 4; ++kk) {
                                constexpr float4_t zero4 = {0.f, 0.f, 0.f, 0.f};
                                const bool first = (kk & LAST) == 0;
                                const half8_t af = __builtin_bit_cast(
                                    half8_t, abase_t[tm * 16 * kLdaVec + 4 * kk]);
#pragma unroll
                                for (int tn = 0; tn < TN; ++tn)
                                    d[tn] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                                        af, bq[tn][kk], first ? zero4 : d[tn], 0, 0, 0);
                                xs = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                                    af, ones, first ? zero4 : xs, 0, 0, 0);
                                if ((kk & LAST) == LAST) {
#pragma unroll
                                    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
                                        for (int r = 0; r < 4; ++r)
                                            acc[tm][tn][r] = fmaf(
                                                ck[tn][kk], xs[r],
                                                fmaf(sk[tn][kk], d[tn][r], acc[tm][tn][r]));
                                }
                            }
                        }
                    };
                    if (gshift == 0)
                        groups(std::integral_constant<int, 0>{});
                    else
                        groups(std::integral_constant<int, 1>{});
                }
            };
            mma(clamp);
        } else {
            // B fragments of this wave's group: [tn][kk]
            auto mma = [&](auto clamp) __attribute__((always_inline)) {
                half8_t bf[TN][4];
#pragma unroll
                for (int tn = 0; tn < TN; ++tn) {
                    const _Float16 sh = __builtin_bit_cast(_Float16, (uint16_t)cur.s[tn]);
                    const half2_t s2 = {sh, sh};
                    const uint32_t words[4] = {cur.w[tn].x, cur.w[tn].y, cur.w[tn].z,
                                               cur.w[tn].w};
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
                for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
                    for (int tm = 0; tm < TM; ++tm) {
                        const uint4 av = abase[tm * 16 * kLdaVec + kk];
                        const half8_t af = __builtin_bit_cast(half8_t, av);
#pragma unroll
                        for (int tn = 0; tn < TN; ++tn)
                            acc[tm][tn] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                                af, bf[tn][kk], acc[tm][tn], 0, 0, 0);
                    }
                }
            };
            mma(clamp);
        }
        if (step + 1 < nsteps) {
            store_a((step + 1) & 1, a_regs);
            store_s((step + 1) & 1);
            if (step + 2 < nsteps) {
                load_a(step + 2, a_regs);
                load_s(step + 2);
                load_b(step + 2, cur);    // cur is consumed; it next serves step s + 2
            }
        }
        __syncthreads();
    };

    // Does any row of this block need the slow copy of the K loop?  For
    // symmetric weights: a group whose scale reaches 9360, the one case where
    // fp16(s * q) can overflow.  For asymmetric weights: a scale of 64 or
    // more (s * (n - z) may then leave the fp16 range) or a zero point
    // beyond +-1000 (codes n - z no longer exact in fp16).  The block's scales (and
    // zero points) are one contiguous span each, scanned once; the K loop
    // below exists in two copies and the common one carries no check.
    constexpr uint32_t kSlowScale = ASYM ? 0x5400u : kHugeScaleBits;   // 64 : 9360
    bool huge = false;
    {
        // the scanned columns: the block's own, or (PART 2) the scan_bn
        // columns of the block tile it completes
        const int n_scan = PART == 2 ? n_blk / scan_bn * scan_bn : n_blk;
        const int scan_w = PART == 2 ? scan_bn : BN;
        const uint32_t span = (uint32_t)min(scan_w, N - n_scan) * srow;
        const __amdgpu_buffer_rsrc_t ssr =
            PART == 2 ? buffer_rsrc(reinterpret_cast<const char*>(scales) + (size_t)n_scan * srow,
                                    (uint64_t)(N - n_scan) * srow)
                      : sr;
        const __amdgpu_buffer_rsrc_t szr =
            PART == 2 && ASYM
                ? buffer_rsrc(reinterpret_cast<const char*>(zeros) + (size_t)n_scan * srow,
                              (uint64_t)(N - n_scan) * srow)
                : zr;
        auto slow_z = [&](uint32_t zbits) {
            const int z = (int)(int16_t)(uint16_t)zbits;
            return ASYM && (z > kZeroClamp || z < -kZeroClamp);
        };
        if ((reinterpret_cast<uintptr_t>(scales) & 15) == 0 &&
            (!ASYM || (reinterpret_cast<uintptr_t>(zeros) & 15) == 0) && (srow & 15) == 0) {
            for (uint32_t off = threadIdx.x * 16u; off < span; off += NT * 16u) {
                const v4u v = __builtin_amdgcn_raw_buffer_load_b128(ssr, off, 0, 0);
                const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    huge |= (w[i] & 0xFFFFu) >= kSlowScale || (w[i] >> 16) >= kSlowScale;
                if constexpr (ASYM) {
                    const v4u zv = __builtin_amdgcn_raw_buffer_load_b128(szr, off, 0, 0);
                    const uint32_t zw[4] = {zv.x, zv.y, zv.z, zv.w};
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        huge |= slow_z(zw[i] & 0xFFFFu) || slow_z(zw[i] >> 16);
                }
            }
        } else {
            for (uint32_t off = threadIdx.x * 2u; off < span; off += NT * 2u) {
                huge |= __builtin_amdgcn_raw_buffer_load_b16(ssr, off, 0, 0) >= kSlowScale;
                if constexpr (ASYM) huge |= slow_z(__builtin_amdgcn_raw_buffer_load_b16(szr, off, 0, 0));
            }
        }
    }
    // block-wide OR of the scan: one word per wave, read after the barrier
    __shared__ uint32_t huge_waves[NT / kWave];
    auto block_any = [&](bool v) {
        const bool wave_v = __any(v);
        if (lane == 0) huge_waves[wave] = wave_v ? 1u : 0u;
        __syncthreads();
        bool any = false;
#pragma unroll
        for (int w = 0; w < NT / kWave; ++w) any |= huge_waves[w] != 0u;
        return any;
    };
    // the slow-only launch decides before loading anything: most blocks leave
    if constexpr (PART == 2) {
        if (!block_any(huge)) return;
    }

    load_a(0, a_regs);
    load_s(0);
    load_b(0, b0);
    store_a(0, a_regs);
    store_s(0);
    if (nsteps > 1) {
        load_a(1, a_regs);
        load_s(1);
        load_b(1, b1);
    }
    if constexpr (PART != 2) {
        huge = block_any(huge);
        if (PART == 1 && huge) return;       // left to the slow-only launch
    } else {
        __syncthreads();                     // the stage-0 A tile is in LDS
    }
    auto k_loop = [&](auto clamp) __attribute__((always_inline)) {
        for (int step = 0; step < nsteps; step += 2) {
            step_body(step, b0, clamp);
            if (step + 1 < nsteps) step_body(step + 1, b1, clamp);
        }
    };
    // one call site per instantiation, so each copy is inlined (a lambda
    // called from two sites can stay a call, with its captured arrays in
    // scratch memory)
    if constexpr (PART == 1)
        k_loop(std::false_type{});
    else if constexpr (PART == 2)
        k_loop(std::true_type{});
    else if (huge)
        k_loop(std::true_type{});
    else
        k_loop(std::false_type{});

    if constexpr (WK > 1) {
        // Sum the WK partial tiles: waves wk > 0 publish, wave wk == 0 adds.
        float4_t* red = reinterpret_cast<float4_t*>(lds);
        const int tile = wm * WN + wn;
        if (wk > 0) {
#pragma unroll
            for (int tm = 0; tm < TM; ++tm)
#pragma unroll
                for (int tn = 0; tn < TN; ++tn)
                    red[(((wk - 1) * WM * WN + tile) * TM * TN + tm * TN + tn) * 64 + lane] =
                        acc[tm][tn];
        }
        __syncthreads();
        if (wk > 0) return;
#pragma unroll
        for (int w = 1; w < WK; ++w)
#pragma unroll
            for (int tm = 0; tm < TM; ++tm)
#pragma unroll
                for (int tn = 0; tn < TN; ++tn)
                    acc[tm][tn] += red[(((w - 1) * WM * WN + tile) * TM * TN + tm * TN + tn) * 64 +
                                       lane];
    }

    if constexpr (SPLIT) {
        // This slice's partial tile goes to the workspace in the lanes' own
        // layout (slice ks of tile t at float4 (t ksplit + ks) PT); the
        // second kernel, split_sum_kernel, adds the slices once the grid has
        // completed.
        constexpr int PT = WM * WN * TM * TN * kWave;     // float4 per block partial
        const int tile = (int)(blockIdx.y * gridDim.x + blockIdx.x);
        const int ks = (int)blockIdx.z;
        const __amdgpu_buffer_rsrc_t wsr = buffer_rsrc(
            partials + (size_t)tile * ksplit * PT, (uint64_t)ksplit * PT * sizeof(float4_t));
        const int wt = wm * WN + wn;
#pragma unroll
        for (int tm = 0; tm < TM; ++tm)
#pragma unroll
            for (int tn = 0; tn < TN; ++tn) {
                const uint32_t off =
                    (uint32_t)((ks * PT + ((wt * TM + tm) * TN + tn) * kWave + lane) * 16);
                const v4u v = {__float_as_uint(acc[tm][tn][0]), __float_as_uint(acc[tm][tn][1]),
                               __float_as_uint(acc[tm][tn][2]), __float_as_uint(acc[tm][tn][3])};
                __builtin_amdgcn_raw_buffer_store_b128(v, wsr, off, 0, kCoherentSc1);
            }
        return;
    }

#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
            const int n = n_blk + (wn * TN + tn) * 16 + l16;
            if (n >= N) continue;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m_blk + (wm * TM + tm) * 16 + 4 * j + r;
                if (m < M) Y[(size_t)m * N + n] = f32_to_f16_bits(acc[tm][tn][r]);
            }
        }
    }
}

namespace {

template <int TM, int TN, int WM, int WN, int WK, bool ASYM = false, bool SPLIT = false,
          int PART = 0, bool SST = false>
hipError_t launch_mfma_sst(const uint16_t* X, int64_t M, const uint32_t* packed,
                           const uint16_t* scales, int64_t N, int64_t K, uint16_t* Y,
                           hipStream_t stream, int gshift, const int16_t* zeros,
                           const TiledSplit* split, int scan_bn) {
    constexpr int BM = 16 * TM * WM;
    constexpr int BN = 16 * TN * WN;
    const size_t a_bytes = (size_t)2 * WK * BM * kLdaVec * sizeof(uint4);   // two A buffers
    const size_t s_bytes = SST ? (size_t)2 * (ASYM ? 2 : 1) * WK * BN * 2 : 0;   // staged scales
    const size_t red_bytes = (size_t)(WK - 1) * WM * WN * TM * TN * 64 * sizeof(float4_t);
    const size_t lds = a_bytes + s_bytes > red_bytes ? a_bytes + s_bytes : red_bytes;
    auto kern = gemm_mfma_kernel<TM, TN, WM, WN, WK, ASYM, SPLIT, PART, SST>;
    if (lds > 64 * 1024) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 (int)lds);
        if (e != hipSuccess) return e;
    }
    const dim3 grid((unsigned)((N + BN - 1) / BN), (unsigned)((M + BM - 1) / BM),
                    SPLIT ? (unsigned)split->ksplit : 1u);
    hipLaunchKernelGGL(kern, grid, dim3(WM * WN * WK * kWave), lds, stream, X, (int)M,
                       reinterpret_cast<const uint4*>(packed), scales, zeros, Y, (int)N, (int)K,
                       gshift, SPLIT ? split->ksplit : 1, SPLIT ? split->groups_per_slice : 0,
                       SPLIT ? reinterpret_cast<float4_t*>(split->partials) : nullptr, scan_bn);
    return hipGetLastError();
}

// The prefill tiles (more than 64 rows of X) stage the scales through LDS
// for group 128, and the scales and zero points of asymmetric weights for
// every group from 128 up (one scale per step or fewer); smaller groups and
// the few-row tiles load them per lane.  Measured at M = 512 (graph replays,
// bit-identical outputs): asymmetric 4096x14336 76.3 against 85.5 us,
// 14336x4096 107.5 against 110.5 us; symmetric group 128 4096x14336 66.8-67.1
// against 67.4-67.8 us (M = 128: 28.5-29.6 against 30.1-30.3 us); symmetric
// group 256 and per channel 0.5-1.5 % slower, so they keep per-lane loads.
template <int TM, int TN, int WM, int WN, int WK, bool ASYM = false, bool SPLIT = false,
          int PART = 0>
hipError_t launch_mfma_t(const uint16_t* X, int64_t M, const uint32_t* packed,
                         const uint16_t* scales, int64_t N, int64_t K, uint16_t* Y,
                         hipStream_t stream, int gshift, const int16_t* zeros = nullptr,
                         const TiledSplit* split = nullptr, int scan_bn = 0) {
    if constexpr (16 * TM * WM >= 64 && (16 * TN * WN) % kWave == 0) {
        if ((ASYM ? gshift >= 2 : gshift == 2) && M > 64)
            return launch_mfma_sst<TM, TN, WM, WN, WK, ASYM, SPLIT, PART, true>(
                X, M, packed, scales, N, K, Y, stream, gshift, zeros, split, scan_bn);
    }
    return launch_mfma_sst<TM, TN, WM, WN, WK, ASYM, SPLIT, PART, false>(
        X, M, packed, scales, N, K, Y, stream, gshift, zeros, split, scan_bn);
}

// Tile shapes by M for the tiled kernel (the symmetric path sends M <= 64
// to the other kernels first when they apply).
template <bool ASYM>
hipError_t launch_tiled(const uint16_t* X, int64_t M, const uint32_t* packed,
                        const uint16_t* scales, const int16_t* zeros, int64_t N, int64_t K,
                        uint16_t* Y, hipStream_t stream, int num_cu, int gshift) {
    if (K > kTiledMaxK)
        return launch_gemv_valu(X, M, packed, scales, N, K, Y, stream, num_cu, gshift, nullptr,
                                ASYM ? zeros : nullptr);
#define W4A16_TILED(TM, TN, WM, WN, WK) \
    launch_mfma_t<TM, TN, WM, WN, WK, ASYM>(X, M, packed, scales, N, K, Y, stream, gshift, zeros)
    // Few rows: 16, 32 or 64 rows of X per block and waves splitting K.
    // With many columns (N >= 32 per compute unit) two waves across 32
    // columns and four over K; with few (the down projections, K > N) one
    // 16-column tile per block and eight waves over K, so that each wave
    // walks fewer groups (14336 x 4096 at group 32, M = 8: 17.8 us against
    // 26.9 us with four waves; M = 64: 33 us against 106 us with 64 x 64
    // blocks).
    const bool wide = N >= (int64_t)32 * num_cu;
    if (M <= 16) return wide ? W4A16_TILED(1, 1, 1, 2, 4) : W4A16_TILED(1, 1, 1, 1, 8);
    if (M <= 32) return wide ? W4A16_TILED(2, 1, 1, 2, 4) : W4A16_TILED(2, 1, 1, 1, 8);
    if (M <= 64) return wide ? W4A16_TILED(2, 1, 1, 2, 4) : W4A16_TILED(2, 2, 1, 1, 8);
    // Prefill: the largest block tile that still gives about one block per
    // compute unit (7/8 of them).
    auto fills = [&](int64_t bm, int64_t bn) {
        return ((M + bm - 1) / bm) * ((N + bn - 1) / bn) * 8 >= (int64_t)num_cu * 7;
    };
    if constexpr (ASYM) {
        // Asymmetric weights.  The exact slow copy of the loop does not fit
        // two waves per SIMD with 32-column wave tiles, so when 128 x 256
        // blocks fill the compute units the common copy runs alone in them
        // (blocks that need the slow copy return at once) and a second launch
        // of 128 x 128 blocks runs the slow copy where it is needed (its
        // blocks decide over the 256 columns of the first launch's block, so
        // every block is computed once; elsewhere they return before loading
        // anything).  Otherwise 16-column wave tiles with both copies: 128 x
        // 128 blocks, 128 x 64 and 64 x 64 blocks with two waves over K; with
        // one scale per step or fewer (staged through LDS) 64 x 128 blocks of
        // 64 x 32 wave tiles, two waves over K, before 128 x 64 (M = 512:
        // 14336x4096 91.2 against 107.0 us, 18944x3584 125.3 against 143.5,
        // 4096x4096 28.8 against 33.1; at group 32 they were slower, 122
        // against 113 us).
        if (fills(128, 256)) {
            const hipError_t e = launch_mfma_t<8, 2, 1, 8, 1, true, false, 1>(
                X, M, packed, scales, N, K, Y, stream, gshift, zeros);
            if (e != hipSuccess) return e;
            return launch_mfma_t<8, 1, 1, 8, 1, true, false, 2>(
                X, M, packed, scales, N, K, Y, stream, gshift, zeros, nullptr, 256);
        }
        if (fills(128, 128)) return W4A16_TILED(8, 1, 1, 8, 1);
        if (gshift >= 2 && fills(64, 128)) return W4A16_TILED(4, 2, 1, 4, 2);
        if (fills(128, 64)) return W4A16_TILED(8, 1, 1, 4, 2);
        return W4A16_TILED(4, 1, 1, 4, 2);
    } else {
        // 128 x 256 (eight waves across N, 128 x 32 wave tiles), 128 x 128
        // and 64 x 128 (four waves across N, two over K), else 64 x 64 (64 x
        // 16 wave tiles, four across N, two over K).  Measured at M = 512 /
        // 256 / 128 (us): 4096 x 14336 69 / 45 / 29, 14336 x 4096 95 / 68 /
        // 66, 8192 x 28672 264 / 131 / 87, 18944 x 3584 120 / 87 / 88,
        // against 67 / 59 / 34, 107 / 99 / 98, 261 / 131 / 117 and 132 / 130
        // / 131 with the earlier choice between 128 x 256 and 128 x 64
        // blocks.
        if (fills(128, 256)) return W4A16_TILED(8, 2, 1, 8, 1);
        if (fills(128, 128)) return W4A16_TILED(8, 2, 1, 4, 2);
        if (fills(64, 128)) return W4A16_TILED(4, 2, 1, 4, 2);
        return W4A16_TILED(4, 1, 1, 4, 2);
    }
#undef W4A16_TILED
}

}  // namespace

TiledSplit plan_tiled_split(int64_t M, int64_t N, int64_t K, int num_cu, int ksplit, int bm) {
    TiledSplit p{};
    p.ksplit = 1;
    const int64_t ngroups = K / kGroup;
    if (M <= 64 || N < 1 || ngroups < 2 || K > kTiledMaxK || num_cu < 1 || (bm != 64 && bm != 128))
        return p;
    const int64_t tiles = ((M + bm - 1) / bm) * ((N + 255) / 256);
    int64_t s = ksplit;
    if (s <= 0) {
        if (tiles * 8 >= (int64_t)num_cu * 7) return p;          // the tiles fill the CUs
        // slices to give about 7/8 of the compute units a block, each slice
        // at least 8 groups (1024 elements of K) long
        s = ((int64_t)num_cu * 7 + 8 * tiles - 1) / (8 * tiles);
        const int64_t max_s = ngroups / 8;
        if (s > max_s) s = max_s;
    }
    if (s > ngroups) s = ngroups;
    if (s < 2) return p;
    const int64_t gps = (ngroups + s - 1) / s;
    s = (ngroups + gps - 1) / gps;                               // every slice holds a group
    if (s < 2) return p;
    const int64_t partial_bytes = (int64_t)bm * 256 * 4;         // bm x 256 fp32 tile
    p.ksplit = (int)s;
    p.groups_per_slice = (int)gps;
    p.tiles = (int)tiles;
    p.workspace_bytes = (size_t)tiles * s * partial_bytes;
    return p;
}

// Second pass of the K split: one thread per float4 of every partial tile
// (the lanes' layout of the split kernel's stores) adds the slices in slice
// order and writes its four outputs.  The whole grid shares the reads: a
// single-pass form, in which the last slice's block of each tile added the
// others' partials, left them to one compute unit per tile and was slower at
// every slice count (14336x4096, 4 / 7 / 14 slices: 76.9 / 53.5 / 49.2
// against 73.3-74.0 / 46.5 / 32.6 us; outputs bit-identical).
template <int TM, int TN, int WM, int WN>
__global__ __launch_bounds__(256) void split_sum_kernel(const float4_t* __restrict__ partials,
                                                        int ksplit, int ntn,
                                                        uint16_t* __restrict__ Y, int M, int N) {
    constexpr int PT = WM * WN * TM * TN * kWave;     // float4 per partial tile
    static_assert(PT % 256 == 0, "a block covers part of one tile");
    const int tile = (int)blockIdx.x / (PT / 256);
    const int e = ((int)blockIdx.x % (PT / 256)) * 256 + (int)threadIdx.x;
    const int lane = e % kWave;
    const int rest = e / kWave;                       // (wave tile, tm, tn)
    const int tn = rest % TN, tm = (rest / TN) % TM, wt = rest / (TN * TM);
    const int wn = wt % WN, wm = wt / WN;
    const int n = (tile % ntn) * (16 * TN * WN) + (wn * TN + tn) * 16 + (lane & 15);
    const int m0 = (tile / ntn) * (16 * TM * WM) + (wm * TM + tm) * 16 + 4 * (lane >> 4);
    const float4_t* p = partials + (size_t)tile * ksplit * PT + e;
    float4_t acc = {0.f, 0.f, 0.f, 0.f};
    int sl = 0;
    for (; sl + 4 <= ksplit; sl += 4) {
        const float4_t v0 = p[(size_t)sl * PT], v1 = p[(size_t)(sl + 1) * PT];
        const float4_t v2 = p[(size_t)(sl + 2) * PT], v3 = p[(size_t)(sl + 3) * PT];
        acc += v0;
        acc += v1;
        acc += v2;
        acc += v3;
    }
    for (; sl < ksplit; ++sl) acc += p[(size_t)sl * PT];
    if (n >= N) return;
#pragma unroll
    for (int r = 0; r < 4; ++r)
        if (m0 + r < M) Y[(size_t)(m0 + r) * N + n] = f32_to_f16_bits(acc[r]);
}

hipError_t launch_gemm_tiled_split(const uint16_t* X, int64_t M, const uint32_t* packed,
                                   const uint16_t* scales, int64_t N, int64_t K, uint16_t* Y,
                                   hipStream_t stream, int gshift, const TiledSplit& plan,
                                   void* workspace) {
    if (plan.ksplit < 2 || workspace == nullptr) return hipErrorInvalidValue;
    TiledSplit p = plan;
    p.partials = workspace;
    hipError_t e = launch_mfma_t<8, 2, 1, 8, 1, false, true>(X, M, packed, scales, N, K, Y,
                                                             stream, gshift, nullptr, &p);
    if (e != hipSuccess) return e;
    constexpr int PT = 8 * 2 * 1 * 8 * kWave;
    const int ntn = (int)((N + 255) / 256);
    hipLaunchKernelGGL((split_sum_kernel<8, 2, 1, 8>), dim3((unsigned)(p.tiles * (PT / 256))),
                       dim3(256), 0, stream, static_cast<const float4_t*>(p.partials), p.ksplit,
                       ntn, Y, (int)M, (int)N);
    return hipGetLastError();
}

hipError_t launch_gemm_mfma(const uint16_t* X, int64_t M, const uint32_t* packed,
                            const uint16_t* scales, int64_t N, int64_t K, uint16_t* Y,
                            hipStream_t stream, int num_cu, int gshift) {
    // The streaming kernels below read one scale per 128 elements; other
    // groups take the tiled kernel for every M.
    if (gshift == 2) {
        // Up to four rows: the streaming GEMV on 4x4x4 matrix-core blocks
        // while x fits in LDS (K == 0, all outputs zero, stays on the tiled
        // kernel).
        if (M <= kMfma4MaxM && K > 0 && M * K * 2 <= kMfma4MaxXBytes)
            return launch_gemv_mfma4(X, M, packed, scales, N, K, Y, stream, num_cu);
        // Batched decode: blocks own contiguous weight rows, X through LDS.
        if (M <= kBatchedMaxM && K > 0 && K <= kBatchedMaxK)
            return launch_gemm_batched(X, M, packed, scales, N, K, Y, stream, num_cu);
        // Few rows and K > N (few output tiles, long rows): the streaming
        // kernel with the K groups split over waves.
        if (M <= 64 && K > N && K <= kSkinnyMaxK)
            return launch_gemm_skinny(X, M, packed, scales, N, K, Y, stream, num_cu);
    }
    return launch_tiled<false>(X, M, packed, scales, nullptr, N, K, Y, stream, num_cu, gshift);
}

hipError_t launch_gemm_tiled_split_asym(const uint16_t* X, int64_t M, const uint32_t* packed,
                                        const uint16_t* scales, const int16_t* zeros, int64_t N,
                                        int64_t K, uint16_t* Y, hipStream_t stream,
                                        const TiledSplit& plan, void* workspace) {
    // 64 x 256 blocks of 64 x 32 wave tiles: both copies of the asymmetric
    // loop fit two waves per SIMD (the 128 x 256 block's wave tile does not).
    if (plan.ksplit < 2 || workspace == nullptr) return hipErrorInvalidValue;
    TiledSplit p = plan;
    p.partials = workspace;
    hipError_t e = launch_mfma_t<4, 2, 1, 8, 1, true, true>(X, M, packed, scales, N, K, Y, stream,
                                                            2, zeros, &p);
    if (e != hipSuccess) return e;
    constexpr int PT = 4 * 2 * 1 * 8 * kWave;
    const int ntn = (int)((N + 255) / 256);
    hipLaunchKernelGGL((split_sum_kernel<4, 2, 1, 8>), dim3((unsigned)(p.tiles * (PT / 256))),
                       dim3(256), 0, stream, static_cast<const float4_t*>(p.partials), p.ksplit,
                       ntn, Y, (int)M, (int)N);
    return hipGetLastError();
}

hipError_t launch_gemm_mfma_asym(const uint16_t* X, int64_t M, const uint32_t* packed,
                                 const uint16_t* scales, const int16_t* zeros, int64_t N,
                                 int64_t K, uint16_t* Y, hipStream_t stream, int num_cu,
                                 int gshift) {
    // Batched decode: blocks own contiguous weight rows, X through LDS.
    if (gshift == 2 && M <= kBatchedMaxM && K > 0 && K <= kBatchedMaxK)
        return launch_gemm_batched_asym(X, M, packed, scales, zeros, N, K, Y, stream, num_cu);
    return launch_tiled<true>(X, M, packed, scales, zeros, N, K, Y, stream, num_cu, gshift);
}

}  // namespace w4a16

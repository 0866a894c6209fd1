// gemv_q4_0.hip — decode GEMV / small-M VALU GEMM on Q4_0 blocks, and the
// Q4_0 quantizer.
//
// Layout ([QUANT] GGUF section: the type table's Q4_0 entry, 32 elements in
// 18 bytes, symmetric with one scale per block, and its Q4_0 dequantizer):
// each row is K/32 consecutive 18-byte blocks, the fp16 scale d (little-
// endian) followed by 16 code bytes, byte 2+i holding element 2i in its low
// nibble and element 2i+1 in its high nibble as q + 8.  The 16 code bytes of
// a block are exactly the 16-byte chunk of the split layout for the same 32
// elements, so the code trick and dot products are shared with gemv.hip;
// only the way a lane obtains its chunk and scale differs.
//
// Blocks are 18 bytes, so a block's bytes are only 2-byte aligned.  A wave
// reads its 64 blocks of a row step (1152 contiguous bytes) with coalesced,
// 16-byte-aligned loads (word l by lane l, words 64..79 by lanes 0..15),
// writes them to a wave-private LDS window, and each lane reads its block
// back at byte offset o0 + 18 l as five dwords, aligning the code bytes with
// one funnel shift per word.  Loads go through raw buffer resources, so
// words past the end of the matrix read as 0; the buffer holds the blocks
// rounded up to a multiple of 16 bytes, so no word is partly inside it.
//
// Grid and prefetch follow gemv_persistent_kernel: whole-x staging in LDS
// (M * K * 2 bytes within the budget), persistent balanced row groups of R
// rows per wave, the next (row group, step) iteration's loads issued before
// the current one is multiplied.
#include "w4a16_device.h"
#include "w4a16_launch.h"

namespace w4a16 {

namespace {

constexpr int kQ40Bytes = 18;                 // bytes per 32-element block
constexpr int kStepBytes = kWave * kQ40Bytes; // 64 blocks per wave step
constexpr int kWindowWords = 80;              // 16-byte words of a row's LDS window

// One lane's block from the wave's LDS window of a row: its 16 code bytes as
// a uint4 (the split layout's chunk) and its scale bits.  off: byte offset of
// the block in the window (even).
__device__ __forceinline__ uint4 block_from_window(const uint32_t* win, uint32_t off,
                                                   uint16_t& d) {
    const uint32_t D = off >> 2;
    const bool mis = (off & 2u) != 0;          // block starts in the upper half of a dword
    uint32_t dw[5];
#pragma unroll
    for (int i = 0; i < 5; ++i) dw[i] = win[D + i];
    d = (uint16_t)(mis ? (dw[0] >> 16) : (dw[0] & 0xFFFFu));
    // codes start 2 bytes after d: bytes 2.. of dw0 when aligned, dw1 when not
    uint32_t c[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) c[j] = mis ? dw[j + 1] : __builtin_amdgcn_alignbit(dw[j + 1], dw[j], 16);
    return make_uint4(c[0], c[1], c[2], c[3]);
}

}  // namespace

// MMAX: activation rows (M <= MMAX).  R: weight rows per wave.  WAVES:
// waves per block.  XPT: 16-byte x blocks staged per thread.
template <int MMAX, int R, int WAVES, int XPT>
__global__ __launch_bounds__(WAVES * kWave) void gemv_q4_0_kernel(
    const uint16_t* __restrict__ X, int M, const uint8_t* __restrict__ blocks,
    uint16_t* __restrict__ Y, int N, int K) {
    extern __shared__ uint4 lds[];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int nb = K >> 5;                                 // blocks per row
    const int nsteps = (nb + kWave - 1) / kWave;
    const int total_rg = (N + R - 1) / R;
    const int stride_rg = gridDim.x * WAVES;
    const int first_rg = blockIdx.x * WAVES + wave;
    const int my_rg = first_rg < total_rg ? (total_rg - 1 - first_rg) / stride_rg + 1 : 0;
    const int T = my_rg * nsteps;
    const uint32_t row_bytes = (uint32_t)nb * kQ40Bytes;
    // the blocks buffer is rounded up to 16 bytes, so every 16-byte word the
    // loads touch is either wholly inside the resource or wholly outside
    const uint64_t total_bytes = ((uint64_t)N * row_bytes + 15) & ~(uint64_t)15;
    const CodeConsts kc = code_consts();
    uint4* xs = lds;
    uint4* win = lds + MMAX * (K >> 3) + wave * (R * kWindowWords);

    const int xblocks = M * (K >> 3);
    uint4 xr[XPT];
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
        const int e = min((int)threadIdx.x + i * WAVES * kWave, xblocks - 1);
        xr[i] = reinterpret_cast<const uint4*>(X)[e];
    }

    // load cursor (wave-uniform)
    int tl = 0, lrg = first_rg, ls = 0;
    uint32_t lead = 0;                                     // row group start mod 16
    __amdgpu_buffer_rsrc_t br = buffer_rsrc(blocks, 0);
    auto load = [&](uint4 (&a)[R], uint4 (&b)[R], uint32_t (&o0)[R]) {
        if (ls == 0) {
            const bool live = tl < T;
            const uint64_t start = live ? (uint64_t)lrg * R * row_bytes : 0;
            const uint64_t base = start & ~(uint64_t)15;
            lead = (uint32_t)(start - base);
            br = buffer_rsrc(blocks + base, live ? total_bytes - base : 0);
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint32_t S = lead + (uint32_t)r * row_bytes + (uint32_t)ls * kStepBytes;
            o0[r] = S & 15u;
            const uint32_t A = S & ~15u;
            typedef unsigned v4u __attribute__((ext_vector_type(4)));
            const v4u va = __builtin_amdgcn_raw_buffer_load_b128(br, A + 16u * lane, 0, kStreamLoad);
            // words 64..79 by lanes 0..15; the other lanes' offset lies past
            // any resource size (at most 2^32 - 1 bytes), so they fetch nothing
            const uint32_t ob = lane < 16 ? A + 1024u + 16u * lane : 0xFFFFFFF0u;
            const v4u vb = __builtin_amdgcn_raw_buffer_load_b128(br, ob, 0, kStreamLoad);
            a[r] = make_uint4(va.x, va.y, va.z, va.w);
            b[r] = make_uint4(vb.x, vb.y, vb.z, vb.w);
        }
        ++tl;
        if (++ls == nsteps) { ls = 0; lrg += stride_rg; }
    };

    uint4 a0[R], b0[R], a1[R], b1[R];
    uint32_t o0a[R], o0b[R];
    load(a0, b0, o0a);

#pragma unroll
    for (int i = 0; i < XPT; ++i) {
        const int e = (int)threadIdx.x + i * WAVES * kWave;
        if (e < xblocks) xs[e] = pair_block(xr[i].x, xr[i].y, xr[i].z, xr[i].w);
    }
    __syncthreads();

    int crg = first_rg, cs = 0;
    float acc[MMAX][R];
#pragma unroll
    for (int m = 0; m < MMAX; ++m)
#pragma unroll
        for (int r = 0; r < R; ++r) acc[m][r] = 0.0f;

    auto compute = [&](const uint4 (&a)[R], const uint4 (&b)[R], const uint32_t (&o0)[R]) {
        // the wave's window: every lane's reads of the previous step are done
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int r = 0; r < R; ++r) {
            win[r * kWindowWords + lane] = a[r];
            if (lane < 16) win[r * kWindowWords + 64 + lane] = b[r];
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const int c = lane + cs * kWave;
        const bool valid = c < nb;
        const int cx = min(c, nb - 1);
        uint4 w[R];
        float sc[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            uint16_t d;
            w[r] = block_from_window(reinterpret_cast<const uint32_t*>(win + r * kWindowWords),
                                     o0[r] + (uint32_t)kQ40Bytes * lane, d);
            sc[r] = valid ? f16_bits_to_f32(d) : 0.0f;
        }
#pragma unroll
        for (int m = 0; m < MMAX; ++m) {
            if (m >= M) break;
            const uint4* xp = xs + m * (K >> 3) + cx * 4;
            const uint4 x0 = xp[0], x1 = xp[1], x2 = xp[2], x3 = xp[3];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                float part = dot_word(w[r].x, x0, 0.0f, kc);
                part = dot_word(w[r].y, x1, part, kc);
                part = dot_word(w[r].z, x2, part, kc);
                part = dot_word(w[r].w, x3, part, kc);
                acc[m][r] = fmaf(sc[r], part, acc[m][r]);
            }
        }
        if (++cs == nsteps) {
            cs = 0;
#pragma unroll
            for (int m = 0; m < MMAX; ++m) {
                if (m >= M) break;
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const float v = wave_sum_lane63(acc[m][r]);
                    const int row = crg * R + r;
                    if (lane == kWave - 1 && row < N) Y[(size_t)m * N + row] = f32_to_f16_bits(v);
                    acc[m][r] = 0.0f;
                }
            }
            crg += stride_rg;
        }
    };

    // Two register sets: the loads of iteration t + 1 are issued before
    // iteration t is multiplied.  Every load is unconditional (iterations
    // past the wave's work read an empty resource).
    for (int t = 0; t < T; t += 2) {
        load(a1, b1, o0b);
        compute(a0, b0, o0a);
        if (t + 1 >= T) break;
        load(a0, b0, o0a);
        compute(a1, b1, o0b);
    }
}

namespace {

constexpr int kQ40XBudget = 64 * 1024;      // bytes of staged activations

template <int MMAX, int R, int WAVES, int XPT>
hipError_t launch_q4_0_xpt(const uint16_t* X, int64_t M, const uint8_t* blocks, int64_t N,
                           int64_t K, uint16_t* Y, hipStream_t stream, int64_t grid) {
    const size_t lds = (size_t)MMAX * (K / 8) * sizeof(uint4) +
                       (size_t)WAVES * R * kWindowWords * sizeof(uint4);
    auto kern = gemv_q4_0_kernel<MMAX, R, WAVES, XPT>;
    if (lds > 64 * 1024) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(WAVES * kWave), lds, stream, X, (int)M,
                       blocks, Y, (int)N, (int)K);
    return hipGetLastError();
}

template <int MMAX, int R, int WAVES>
hipError_t launch_q4_0_t(const uint16_t* X, int64_t M, const uint8_t* blocks, int64_t N,
                         int64_t K, uint16_t* Y, hipStream_t stream, int num_cu,
                         int blocks_per_cu) {
    // a whole number of blocks per compute unit (as for the split layout)
    const int64_t total_rg = (N + R - 1) / R;
    const int64_t per_cu = (int64_t)num_cu * WAVES;
    int64_t grid = (total_rg + WAVES - 1) / WAVES;
    if (total_rg >= per_cu) {
        const int64_t b = total_rg / per_cu;
        grid = (b > blocks_per_cu ? blocks_per_cu : b) * num_cu;
    }
    const int64_t need = (int64_t)MMAX * (K / 8);
    const int64_t threads = (int64_t)WAVES * kWave;
#define W4A16_Q40(XPT) launch_q4_0_xpt<MMAX, R, WAVES, XPT>(X, M, blocks, N, K, Y, stream, grid)
    if (need <= threads) return W4A16_Q40(1);
    if (need <= 2 * threads) return W4A16_Q40(2);
    if (need <= 4 * threads) return W4A16_Q40(4);
    if (need <= 8 * threads) return W4A16_Q40(8);
    return W4A16_Q40(16);
#undef W4A16_Q40
}

// The launch shapes of the split-layout GEMV: up to 8192 elements per row,
// four waves per block and up to eight blocks per compute unit; longer rows eight
// waves and two blocks.
template <int MMAX>
hipError_t launch_q4_0_m(const uint16_t* X, int64_t M, const uint8_t* blocks, int64_t N,
                         int64_t K, uint16_t* Y, hipStream_t stream, int num_cu) {
    constexpr int R = MMAX >= 4 ? 1 : 2;
    if (K >= 12288) return launch_q4_0_t<MMAX, R, 8>(X, M, blocks, N, K, Y, stream, num_cu, 2);
    return launch_q4_0_t<MMAX, R, 4>(X, M, blocks, N, K, Y, stream, num_cu, 8);
}

}  // namespace

hipError_t launch_gemv_q4_0(const uint16_t* X, int64_t M, const uint8_t* blocks, int64_t N,
                            int64_t K, uint16_t* Y, hipStream_t stream, int num_cu) {
    // rows of X per launch so that they fit the staging budget
    int64_t mm = kQ40XBudget / (K * 2);
    mm = mm >= 8 ? 8 : mm >= 4 ? 4 : mm >= 2 ? 2 : 1;
    for (int64_t m0 = 0; m0 < M; m0 += mm) {
        const int64_t rows = (M - m0 < mm) ? (M - m0) : mm;
        const uint16_t* Xs = X + m0 * K;
        uint16_t* Ys = Y + m0 * N;
        hipError_t e;
        if (rows == 1)
            e = launch_q4_0_m<1>(Xs, rows, blocks, N, K, Ys, stream, num_cu);
        else if (rows == 2)
            e = launch_q4_0_m<2>(Xs, rows, blocks, N, K, Ys, stream, num_cu);
        else if (rows <= 4)
            e = launch_q4_0_m<4>(Xs, rows, blocks, N, K, Ys, stream, num_cu);
        else
            e = launch_q4_0_m<8>(Xs, rows, blocks, N, K, Ys, stream, num_cu);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace w4a16

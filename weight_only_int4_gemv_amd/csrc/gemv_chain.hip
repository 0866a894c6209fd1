// gemv_chain.hip — a dependent sequence of decode GEMVs (M = 1) in one
// persistent launch ([BENCH] §二: a decode step streams every weight matrix
// once, layer after layer; each matrix's input is produced by the one
// before it).
//
// Stage s computes y_s = x_s * W_s^T exactly as w4a16_gemv does (same lane
// split, same arithmetic, same reduction order, so the outputs are
// bit-identical), and x_s may be the output of any earlier stage.  Between
// stages the grid synchronizes through counters in a caller-owned buffer:
//   - a block finishing stage s makes its stores visible (release at agent
//     scope) and adds 1 to counter s;
//   - before staging x_{s+1}, one thread of every block waits (acquire at
//     agent scope) until counter s equals the number of blocks;
//   - the weights of stage s+1 do not depend on stage s, so the prefetch
//     ring keeps loading them across the barrier and HBM stays busy.
// The grid is sized to be co-resident (occupancy-checked on the host); every
// wait is bounded (kSpinLimit polls) and sets an error word instead of
// hanging; once the error word is set no later wait polls again.  The last
// block to finish returns every counter to zero, so the buffer is ready for
// the next call (and for graph replays).
#include "w4a16_device.h"
#include "w4a16_launch.h"

namespace w4a16 {

namespace {
constexpr int kChainR = 2;        // rows per wave
constexpr int kChainP = 1;        // steps in flight (ring of P + 1 slots)
constexpr int kChainWaves = 4;    // waves per block
constexpr uint32_t kSpinLimit = 1u << 20;   // about a second of polling
}  // namespace

__global__ __launch_bounds__(kChainWaves * kWave) void gemv_chain_kernel(ChainArgs a) {
    extern __shared__ uint4 lds[];
    constexpr int R = kChainR, P = kChainP, Q = P + 1, WAVES = kChainWaves;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int G = gridDim.x * WAVES;
    const int first_rg = blockIdx.x * WAVES + wave;
    const CodeConsts kc = code_consts();
    uint32_t* const sync = a.sync;

    struct Geo {
        int nchunks, nsteps, total_rg, T, Tp;
        uint32_t wrow, srow;
    };
    auto geo = [&](int s) {
        Geo g;
        const int K = a.st[s].K, N = a.st[s].N;
        g.nchunks = K >> 5;
        g.nsteps = (g.nchunks + kWave - 1) / kWave;
        g.total_rg = (N + R - 1) / R;
        const int my = first_rg < g.total_rg ? (g.total_rg - 1 - first_rg) / G + 1 : 0;
        g.T = my * g.nsteps;             // this wave's live iterations in stage s
        g.Tp = (g.T + Q - 1) / Q * Q;    // padded to whole rings
        g.wrow = (uint32_t)K / 2;
        g.srow = (uint32_t)K / 64;
        return g;
    };

    // ---- load cursor: (stage lst, iteration lt, row group lrg, step ls)
    int lst = 0, lt = 0, lrg = first_rg, ls = 0;
    Geo lg = geo(0);
    auto skip_empty = [&]() {
        while (lst < a.count && lt == lg.Tp) {
            ++lst;
            lt = 0;
            ls = 0;
            lrg = first_rg;
            if (lst < a.count) lg = geo(lst);
        }
    };
    skip_empty();
    __amdgpu_buffer_rsrc_t wr = buffer_rsrc(a.st[0].packed, 0), sr = buffer_rsrc(a.st[0].scales, 0);
    auto load = [&](uint4 (&wd)[R], uint16_t (&sd)[R]) {
        if (ls == 0) {
            const bool live = lst < a.count && lt < lg.T;
            if (live) {
                const int64_t row0 = (int64_t)lrg * R;
                const int64_t rows_left = (int64_t)a.st[lst].N - row0;
                wr = buffer_rsrc(reinterpret_cast<const char*>(a.st[lst].packed) + row0 * lg.wrow,
                                 (uint64_t)rows_left * lg.wrow);
                sr = buffer_rsrc(reinterpret_cast<const char*>(a.st[lst].scales) + row0 * lg.srow,
                                 (uint64_t)rows_left * lg.srow);
            } else {
                wr = buffer_rsrc(a.st[0].packed, 0);
                sr = buffer_rsrc(a.st[0].scales, 0);
            }
        }
        const int voff_w = lane * 16 + ls * (kWave * 16);
        const int voff_s = (lane >> 2) * 2 + ls * (kWave / 4 * 2);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            typedef unsigned v4u __attribute__((ext_vector_type(4)));
            const v4u v = __builtin_amdgcn_raw_buffer_load_b128(wr, voff_w, r * lg.wrow, kStreamLoad);
            wd[r] = make_uint4(v.x, v.y, v.z, v.w);
            sd[r] = __builtin_amdgcn_raw_buffer_load_b16(sr, voff_s, r * lg.srow, kStreamLoad);
        }
        if (lst < a.count) {
            ++lt;
            if (++ls == lg.nsteps) {
                ls = 0;
                lrg += G;
            }
            skip_empty();
        }
    };

    uint4 w[Q][R];
    uint16_t sb[Q][R];
#pragma unroll
    for (int i = 0; i < P; ++i) load(w[i], sb[i]);

    for (int s = 0; s < a.count; ++s) {
        const Geo g = geo(s);
        const int K = a.st[s].K;
        const int N = a.st[s].N;
        if (s > 0) {
            // wait until every block has finished stage s - 1
            if (threadIdx.x == 0) {
                uint32_t spins = 0;
                // Poll relaxed (an acquire per poll would invalidate the
                // caches every time); one acquire fence once the count is
                // reached.  Once any wait has given up, later ones do not
                // wait again.
                while (__hip_atomic_load(&sync[s - 1], __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT) < gridDim.x &&
                       __hip_atomic_load(&sync[kChainErrWord], __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT) == 0) {
                    if (++spins > kSpinLimit) {
                        __hip_atomic_store(&sync[kChainErrWord], 1u, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
                        break;
                    }
                    __builtin_amdgcn_s_sleep(2);
                }
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            }
            __syncthreads();
        }
        // stage x_s (possibly an earlier stage's output) into LDS
        {
            const uint4* xs = reinterpret_cast<const uint4*>(a.st[s].x);
            const int nblk = K >> 3;
            for (int i0 = threadIdx.x; i0 < nblk; i0 += 4 * WAVES * kWave) {
                uint4 v[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int i = i0 + j * WAVES * kWave;
                    if (i < nblk) v[j] = xs[i];
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int i = i0 + j * WAVES * kWave;
                    if (i < nblk) lds[i] = pair_block(v[j].x, v[j].y, v[j].z, v[j].w);
                }
            }
        }
        __syncthreads();

        int crg = first_rg, cs = 0;
        float acc[R];
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] = 0.0f;
        uint16_t* const y = a.st[s].y;
        for (int t0 = 0; t0 < g.Tp; t0 += Q) {
#pragma unroll
            for (int i = 0; i < Q; ++i) {
                load(w[(i + P) % Q], sb[(i + P) % Q]);
                const int c = lane + cs * kWave;
                const bool valid = c < g.nchunks;
                const int cx = min(c, g.nchunks - 1);
                if (t0 + i < g.T) {
                    const uint4* xp = lds + cx * 4;
                    const uint4 x0 = xp[0], x1 = xp[1], x2 = xp[2], x3 = xp[3];
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        float part = dot_word(w[i][r].x, x0, 0.0f, kc);
                        part = dot_word(w[i][r].y, x1, part, kc);
                        part = dot_word(w[i][r].z, x2, part, kc);
                        part = dot_word(w[i][r].w, x3, part, kc);
                        const float sc = valid ? f16_bits_to_f32(sb[i][r]) : 0.0f;
                        acc[r] = fmaf(sc, part, acc[r]);
                    }
                }
                if (++cs == g.nsteps) {
                    cs = 0;
                    if (t0 + i < g.T) {
#pragma unroll
                        for (int r = 0; r < R; ++r) {
                            const float v = wave_sum_lane63(acc[r]);
                            const int row = crg * R + r;
                            if (lane == kWave - 1 && row < N) y[row] = f32_to_f16_bits(v);
                            acc[r] = 0.0f;
                        }
                    }
                    crg += G;
                }
            }
        }
        // this block is done with stage s
        __syncthreads();
        if (threadIdx.x == 0)
            __hip_atomic_fetch_add(&sync[s], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    }

    // The last block out returns the counters to zero.
    if (threadIdx.x == 0) {
        const uint32_t prev = __hip_atomic_fetch_add(&sync[kChainDoneWord], 1u, __ATOMIC_ACQ_REL,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        if (prev == gridDim.x - 1) {
            for (int s = 0; s < a.count; ++s)
                __hip_atomic_store(&sync[s], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&sync[kChainDoneWord], 0u, __ATOMIC_RELEASE,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

hipError_t launch_gemv_chain(const ChainArgs& args, int64_t max_k, hipStream_t stream,
                             int num_cu, int* blocks_out) {
    const size_t lds = (size_t)(max_k / 8) * sizeof(uint4);
    int occ = 0;
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &occ, reinterpret_cast<const void*>(gemv_chain_kernel), kChainWaves * kWave, lds);
    if (e != hipSuccess) return e;
    // co-resident grid: the blocks wait on each other
    const int per_cu = occ < 4 ? occ : 4;
    if (per_cu < 1) return hipErrorInvalidConfiguration;
    const int blocks = per_cu * num_cu;
    if (blocks_out) *blocks_out = blocks;
    hipLaunchKernelGGL(gemv_chain_kernel, dim3(blocks), dim3(kChainWaves * kWave), lds, stream,
                       args);
    return hipGetLastError();
}

}  // namespace w4a16

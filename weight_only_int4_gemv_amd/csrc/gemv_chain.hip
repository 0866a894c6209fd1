// gemv_chain.hip — a dependent sequence of decode GEMVs (M = 1) in one
// persistent launch ([BENCH] §二: a decode step streams every weight matrix
// once, layer after layer; each matrix's input is produced by the one
// before it).
//
// Stage s computes y_s = x_s * W_s^T exactly as w4a16_gemv does (same lane
// split — 64 lanes per row, or 16 with four rows side by side where
// gemv_lanes_per_row says so —, same arithmetic, same reduction order, so
// the outputs are bit-identical), and x_s may be the output of any earlier
// stage.
//
// One block per compute unit: W compute waves and C control waves.
//   - Compute waves stream the weights of all stages through one ring of
//     P + 1 register slots that runs across stage boundaries, so the loads of
//     the next stages are in flight while the grid synchronizes.  A finished
//     row's output goes to LDS, not to memory.  Compute waves issue no other
//     memory loads: a wait for one (the vector memory counter is in order)
//     would also wait for every weight load issued before it.
//   - The first control wave, once the block's compute waves have finished
//     stage s - 1, writes the block's outputs of that stage to memory with
//     stores coherent at device scope (they write through the per-XCD L2),
//     waits for them to complete, arrives on a two-level counter tree (eight
//     leaves, then a root), and waits for the root to count every block.
//   - Then the control waves read x_s with device-coherent loads (stale
//     lines in an XCD's L2 are never used) into LDS, and the compute waves
//     start stage s.
// Cross-block data is only ever written and read with device-coherent
// accesses, so no cache write-back or invalidate is needed: the control
// wave's wait for its stores' completion orders them before its arrival.
// Every wait is bounded (kSpinLimit polls) and sets the error word instead
// of hanging; once the error word is set no later wait polls again.  The
// last block to finish returns every counter to zero, so the buffer is ready
// for the next call (and for graph replays).
#include <mutex>

#include "w4a16_device.h"
#include "w4a16_launch.h"

namespace w4a16 {

namespace {
constexpr int kChainR = 2;                 // rows per wave and row group
constexpr uint32_t kSpinLimit = 1u << 20;  // about a second of polling
constexpr int kCoherent = 16;              // cache policy: coherent at device scope (sc1)
constexpr int kRootWord = kChainLineWords;
constexpr int kLeafWord0 = 2 * kChainLineWords;
constexpr int kDoneWord = (2 + kChainLeaves) * kChainLineWords;

__device__ __forceinline__ uint32_t sync_load(uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void sync_store(uint32_t* p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t sync_add(uint32_t* p, uint32_t v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Block barrier without a memory fence: LDS writes are waited for
// explicitly (lgkmcnt) by the waves that made them; outstanding weight loads
// are not waited for.  The empty asm keeps the compiler from moving memory
// accesses across it.
__device__ __forceinline__ void block_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}
// s_waitcnt through the builtin (not inline asm), so that the compiler's
// own wait tracking knows what has completed.  gfx9 encoding: vmcnt in bits
// 3:0 and 15:14, expcnt in 6:4, lgkmcnt in 11:8.
__device__ __forceinline__ void wait_lds() {
    __builtin_amdgcn_s_waitcnt(0xC07F);    // lgkmcnt(0)
}
__device__ __forceinline__ void wait_vmem() {
    __builtin_amdgcn_s_waitcnt(0x0F70);    // vmcnt(0)
}
}  // namespace

template <int W, int C, int P>
__global__ __launch_bounds__((W + C) * kWave) void gemv_chain_kernel(ChainArgs a, int ycap) {
    extern __shared__ uint4 lds[];
    constexpr int R = kChainR, Q = P + 1;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int G = gridDim.x * W;                       // compute waves in the grid
    uint32_t* const sync = a.sync;
    uint16_t* const ybuf = reinterpret_cast<uint16_t*>(lds + a.x_vecs);   // [W][ycap]

    struct Geo {
        int nchunks, nsteps, total_rg, T;
        int lpr, sh, S, RG;       // lanes per row (1 << sh), rows side by side, rows a group
        uint32_t wrow, srow;
    };
    auto geo = [&](int s, int first_rg) {
        Geo g;
        const int K = a.st[s].K, N = a.st[s].N;
        g.nchunks = K >> 5;
        g.lpr = gemv_lanes_per_row(K, N, gridDim.x);    // as w4a16_gemv (one block per CU)
        g.sh = g.lpr == 16 ? 4 : 6;
        g.S = kWave / g.lpr;
        g.RG = R * g.S;
        g.nsteps = (g.nchunks + g.lpr - 1) / g.lpr;
        g.total_rg = (N + g.RG - 1) / g.RG;
        const int my = first_rg < g.total_rg ? (g.total_rg - 1 - first_rg) / G + 1 : 0;
        g.T = my * g.nsteps;             // the wave's iterations in stage s
        g.wrow = (uint32_t)K / 2;
        g.srow = (uint32_t)K / 64;
        return g;
    };

    if (wave >= W) {
        // ------------------------------------------------ control waves
        const bool syncer = wave == W;
        const int ctid = (int)threadIdx.x - W * kWave;     // 0 .. C*64-1
        const int leaf = blockIdx.x % kChainLeaves;
        const uint32_t per_leaf = gridDim.x / kChainLeaves;
        auto flush = [&](int s) {
            // outputs of stage s held in LDS -> y_s, device-coherent stores
            const Geo g = geo(s, 0);
            const int my_max = (g.total_rg + G - 1) / G;
            const int per_wave = my_max * g.RG;
            const __amdgpu_buffer_rsrc_t yr = buffer_rsrc(a.st[s].y, (uint64_t)a.st[s].N * 2);
            for (int e = lane; e < W * per_wave; e += kWave) {
                const int w = e / per_wave;
                const int jr = e - w * per_wave;
                const int i = jr / g.RG;
                const int r = jr - i * g.RG;            // row within the group
                const int rg = blockIdx.x * W + w + i * G;
                if (rg < g.total_rg) {
                    const int row = rg * g.RG + r;
                    __builtin_amdgcn_raw_buffer_store_b16(ybuf[w * ycap + jr], yr, row * 2, 0,
                                                          kCoherent);
                }
            }
            wait_vmem();   // the stores are complete (visible to every XCD)
        };
        for (int s = 0; s < a.count; ++s) {
            if (s > 0) {
                block_barrier();                                   // B1: stage s-1 outputs in LDS
                if (syncer) {
                    flush(s - 1);
                    if (lane == 0) {
                        const uint32_t old =
                            sync_add(&sync[kLeafWord0 + leaf * kChainLineWords], 1u);
                        if (old == (uint32_t)s * per_leaf - 1) sync_add(&sync[kRootWord], 1u);
                        uint32_t spins = 0;
                        while (sync_load(&sync[kRootWord]) < (uint32_t)s * kChainLeaves) {
                            if (sync_load(&sync[kChainErrWord]) != 0) break;
                            if (++spins > kSpinLimit) {
                                sync_store(&sync[kChainErrWord], 1u);
                                break;
                            }
                            __builtin_amdgcn_s_sleep(1);
                        }
                    }
                }
            }
            block_barrier();                                       // B2: x_s may be read
            // x_s -> LDS in the paired order, device-coherent loads in
            // batches of kXBatch per lane
            constexpr int kXBatch = 8;
            const int nblk = a.st[s].K >> 3;
            const __amdgpu_buffer_rsrc_t xr = buffer_rsrc(a.st[s].x, (uint64_t)a.st[s].K * 2);
            for (int i0 = ctid; i0 < nblk; i0 += kXBatch * C * kWave) {
                typedef unsigned v4u __attribute__((ext_vector_type(4)));
                v4u v[kXBatch];
#pragma unroll
                for (int j = 0; j < kXBatch; ++j)
                    v[j] = __builtin_amdgcn_raw_buffer_load_b128(xr, (i0 + j * C * kWave) * 16, 0,
                                                                 kCoherent);
#pragma unroll
                for (int j = 0; j < kXBatch; ++j) {
                    const int i = i0 + j * C * kWave;
                    if (i < nblk) lds[i] = pair_block(v[j].x, v[j].y, v[j].z, v[j].w);
                }
            }
            wait_vmem();
            wait_lds();
            block_barrier();                                       // B3: x_s is in LDS
        }
        block_barrier();                                           // B1 of the last stage
        if (syncer) {
            flush(a.count - 1);
            if (lane == 0) {
                const uint32_t prev = sync_add(&sync[kDoneWord], 1u);
                if (prev == gridDim.x - 1) {
                    // every wait of this call is over: hand its error word to
                    // the caller's status word and clear it, when asked to
                    if (a.status != nullptr) {
                        sync_store(a.status, sync_load(&sync[kChainErrWord]));
                        sync_store(&sync[kChainErrWord], 0u);
                    }
                    // every block is past every wait: return the counters to zero
                    sync_store(&sync[kRootWord], 0u);
                    for (int l = 0; l < kChainLeaves; ++l)
                        sync_store(&sync[kLeafWord0 + l * kChainLineWords], 0u);
                    sync_store(&sync[kDoneWord], 0u);
                }
            }
        }
        return;
    }

    // ---------------------------------------------------- compute waves
    const int first_rg = blockIdx.x * W + wave;
    const CodeConsts kc = code_consts();

    // load cursor: (stage lst, iteration lt in the stage, row group lrg, step ls)
    int lst = 0, lt = 0, lrg = first_rg, ls = 0;
    Geo lg = geo(0, first_rg);
    auto skip_empty = [&]() {
        while (lst < a.count && lt == lg.T) {
            ++lst;
            lt = 0;
            ls = 0;
            lrg = first_rg;
            if (lst < a.count) lg = geo(lst, first_rg);
        }
    };
    skip_empty();
    int total_T = 0;
    for (int s = 0; s < a.count; ++s) total_T += geo(s, first_rg).T;

    const __amdgpu_buffer_rsrc_t empty_w = buffer_rsrc(a.st[0].packed, 0);
    const __amdgpu_buffer_rsrc_t empty_s = buffer_rsrc(a.st[0].scales, 0);
    __amdgpu_buffer_rsrc_t wr = empty_w, sr = empty_s;
    auto load = [&](uint4 (&wd)[R], uint16_t (&sd)[R]) {
        if (ls == 0) {
            if (lst < a.count) {
                const int64_t row0 = (int64_t)lrg * lg.RG;
                const int64_t rows_left = (int64_t)a.st[lst].N - row0;
                wr = buffer_rsrc(reinterpret_cast<const char*>(a.st[lst].packed) + row0 * lg.wrow,
                                 (uint64_t)rows_left * lg.wrow);
                sr = buffer_rsrc(reinterpret_cast<const char*>(a.st[lst].scales) + row0 * lg.srow,
                                 (uint64_t)rows_left * lg.srow);
            } else {
                wr = empty_w;
                sr = empty_s;
            }
        }
        const uint32_t wrow = lst < a.count ? lg.wrow : 0u;
        const uint32_t srow = lst < a.count ? lg.srow : 0u;
        // row r * S + seg of the group (seg in the lane offset), chunk li + ls * lpr
        const int seg = lane >> lg.sh, c = (lane & (lg.lpr - 1)) + ls * lg.lpr;
        const int voff_w = seg * (int)wrow + c * 16;
        const int voff_s = seg * (int)srow + (c >> 2) * 2;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            typedef unsigned v4u __attribute__((ext_vector_type(4)));
            const v4u v = __builtin_amdgcn_raw_buffer_load_b128(wr, voff_w, r * lg.S * wrow,
                                                                 kStreamLoad);
            wd[r] = make_uint4(v.x, v.y, v.z, v.w);
            sd[r] = __builtin_amdgcn_raw_buffer_load_b16(sr, voff_s, r * lg.S * srow, kStreamLoad);
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

    // Stage entry: pass the block barriers of every stage up to s (stages
    // where this wave has no rows included); the control waves put x_t into
    // LDS between B2 and B3.
    int entered = -1;
    auto enter = [&](int s) {
        while (entered < s) {
            const int t = ++entered;
            if (t > 0) {
                wait_lds();
                block_barrier();                                   // B1
            }
            block_barrier();                                       // B2
            block_barrier();                                       // B3
        }
    };

    uint4 w[Q][R];
    uint16_t sb[Q][R];
#pragma unroll
    for (int i = 0; i < P; ++i) load(w[i], sb[i]);

    // compute cursor: stage cst, row group crg, step cs, row-group ordinal j
    int cst = 0, crg = first_rg, cs = 0, cj = 0, ct = 0;
    Geo cg = geo(0, first_rg);
    while (cst < a.count && cg.T == 0) {
        ++cst;
        if (cst < a.count) cg = geo(cst, first_rg);
    }
    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.0f;

    for (int t0 = 0; t0 < total_T; t0 += Q) {
#pragma unroll
        for (int i = 0; i < Q; ++i) {
            load(w[(i + P) % Q], sb[(i + P) % Q]);
            if (t0 + i < total_T) {                                // wave-uniform
                enter(cst);
                const int seg = lane >> cg.sh, li = lane & (cg.lpr - 1);
                const int c = li + cs * cg.lpr;
                const bool valid = c < cg.nchunks;
                const int cx = min(c, cg.nchunks - 1);
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
                if (++cs == cg.nsteps) {
                    // row group complete: reduce over the wave, keep in LDS
                    cs = 0;
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        const float v = cg.lpr == kWave ? wave_sum_lane63(acc[r])
                                                        : row16_sum(acc[r]);
                        if (li == cg.lpr - 1)
                            ybuf[wave * ycap + cj * cg.RG + r * cg.S + seg] = f32_to_f16_bits(v);
                        acc[r] = 0.0f;
                    }
                    ++cj;
                    crg += G;
                    if (++ct == cg.T / cg.nsteps) {
                        // this wave's rows of stage cst are done
                        ct = 0;
                        cj = 0;
                        crg = first_rg;
                        do {
                            ++cst;
                            if (cst < a.count) cg = geo(cst, first_rg);
                        } while (cst < a.count && cg.T == 0);
                    }
                }
            }
        }
    }
    enter(a.count - 1);       // barriers of trailing stages without rows here
    wait_lds();
    block_barrier();          // B1 of the last stage
}

template <int W, int C, int P>
hipError_t launch_chain_t(const ChainArgs& args, int64_t max_n, hipStream_t stream, int num_cu,
                          int* blocks_out) {
    // rows of a stage a wave finishes before its block writes them: the most
    // row groups any wave gets, times the rows of a group (as the kernel's
    // geometry: 2 rows a group, times 4 where 16 lanes share a row)
    const int G = num_cu * W;
    int ycap = 0;
    for (int s = 0; s < args.count; ++s) {
        const int64_t rgsz =
            (int64_t)kChainR * (kWave / gemv_lanes_per_row(args.st[s].K, args.st[s].N, num_cu));
        const int64_t rgs = (args.st[s].N + rgsz - 1) / rgsz;
        const int64_t rows = (rgs + G - 1) / G * rgsz;
        if (rows > ycap) ycap = (int)rows;
    }
    (void)max_n;
    const size_t lds = (size_t)args.x_vecs * sizeof(uint4) + (size_t)W * ycap * 2;
    if (lds > 160 * 1024) return hipErrorInvalidValue;
    int occ = 0;
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &occ, reinterpret_cast<const void*>(gemv_chain_kernel<W, C, P>), (W + C) * kWave, lds);
    if (e != hipSuccess) return e;
    // co-resident grid of one block per compute unit: the blocks wait on
    // each other
    if (occ < 1 || num_cu % kChainLeaves != 0) return hipErrorInvalidConfiguration;
    if (blocks_out) *blocks_out = num_cu;
    hipLaunchKernelGGL((gemv_chain_kernel<W, C, P>), dim3(num_cu), dim3((W + C) * kWave), lds,
                       stream, args, ycap);
    return hipGetLastError();
}

hipError_t launch_gemv_chain(const ChainArgs& args, int64_t max_n, hipStream_t stream, int num_cu,
                             int* blocks_out) {
    // 12 compute + 4 control waves, 4 iterations in flight: the fastest of
    // the shapes measured on the LLaMA-3-8B decode sweep.
    return launch_chain_t<12, 4, 4>(args, max_n, stream, num_cu, blocks_out);
}

// ---------------------------------------------------------------------
// Counters for callers that cannot allocate device memory: one array per
// device, loaded zeroed with the library and returned to zero by every call
// (the last block clears the counters and, because args.status is set, the
// error word).  The array's name is only a host-side handle: its device
// address is looked up once per device and only that address is used.
namespace {
static __device__ __align__(256) uint32_t scratch[kChainSyncWords];

constexpr int kMaxScratchDevices = 64;
uint32_t* g_scratch[kMaxScratchDevices];
std::mutex g_scratch_mutex;

hipError_t scratch_address(int device, uint32_t** out) {
    if (device < 0 || device >= kMaxScratchDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch[device] == nullptr) {
        // `device` is the current device: the lookup returns its copy
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_scratch[device] = static_cast<uint32_t*>(p);
    }
    *out = g_scratch[device];
    return hipSuccess;
}
}  // namespace

hipError_t launch_gemv_chain_noalloc(ChainArgs& args, int64_t max_n, hipStream_t stream,
                                     int num_cu, int device) {
    if (args.status == nullptr) return hipErrorInvalidValue;
    uint32_t* sync = nullptr;
    const hipError_t e = scratch_address(device, &sync);
    if (e != hipSuccess) return e;
    args.sync = sync;
    return launch_chain_t<12, 4, 4>(args, max_n, stream, num_cu, nullptr);
}

}  // namespace w4a16

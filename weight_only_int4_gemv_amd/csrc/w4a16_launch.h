// w4a16_launch.h — host-side launchers of the W4A16 kernels (private).
// Shapes are validated by the C ABI (api.hip) before any of these is called:
// 0 < M, N <= 2^24, 0 <= K < 2^31, K % 128 == 0, pointers aligned.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a16 {

// Group size meaning one scale per row (per channel): the whole row of K.
constexpr int64_t kPerChannel = -1;
// log2(group / 32) handed to the linear-layer kernels for per-channel
// scales: every 32-code chunk of a row maps to scale 0 of the row.
constexpr int kPerChannelShift = 30;
// Scales per row of a layer with chunk shift gshift (one scale per
// 2^gshift chunks of 32 codes; 1 for per-channel scales).
__host__ __device__ inline int scales_per_row(int64_t K, int gshift) {
    return gshift >= kPerChannelShift ? 1 : (int)(K >> (5 + gshift));
}

// group: 32, 64, 128 or 256 elements per scale, or kPerChannel.  perm: NULL, or device
// int32 [K] (column j of the result is column perm[j] of W).  zeros: NULL
// for the symmetric quantizer, or int16 [N, K/group] for the asymmetric one.
hipError_t launch_quantize(const uint16_t* W, int64_t N, int64_t K, int64_t group,
                           uint32_t* packed, uint16_t* scales, hipStream_t stream, int num_cu,
                           const int* perm = nullptr, int16_t* zeros = nullptr);

// Q4_0 blocks: N rows of K/32 blocks of 18 bytes (fp16 d, then 16 code
// bytes) in a buffer rounded up to 16 bytes; `blocks` 16-byte aligned.  The
// GEMV stages x whole in LDS: 0 < K <= kQ40MaxK.
constexpr int64_t kQ40MaxK = 32768;
hipError_t launch_quantize_q4_0(const uint16_t* W, int64_t N, int64_t K, uint8_t* blocks,
                                hipStream_t stream);
hipError_t launch_gemv_q4_0(const uint16_t* X, int64_t M, const uint8_t* blocks, int64_t N,
                            int64_t K, uint16_t* Y, hipStream_t stream, int num_cu);

// VALU dot-product path, any M (M > 8 runs in slices of 8 rows).  gshift:
// log2(group / 32), one scale per 2^gshift 32-code chunks (2 = group 128).
// perm (device int32 [K], 16-byte aligned, or NULL): the weight's columns
// are in the order perm, so column j meets activation X[m, perm[j]].
// zeros (device int16 [N, K/group], or NULL): asymmetric weights, nibbles n
// in [0, 15] and w = s (n - z); NULL: symmetric, w = s (n - 8).
hipError_t launch_gemv_valu(const uint16_t* X, int64_t M, const uint32_t* packed,
                            const uint16_t* scales, int64_t N, int64_t K, uint16_t* Y,
                            hipStream_t stream, int num_cu, int gshift = 2,
                            const int* perm = nullptr, const int16_t* zeros = nullptr);

// MFMA path, any M.  gshift: log2(group / 32) as for launch_gemv_valu; the
// streaming kernels (mfma4, batched, skinny) take group 128 (gshift 2),
// every group runs on the tiled kernel.
hipError_t launch_gemm_mfma(const uint16_t* X, int64_t M, const uint32_t* packed,
                            const uint16_t* scales, int64_t N, int64_t K, uint16_t* Y,
                            hipStream_t stream, int num_cu, int gshift = 2);

// MFMA path for asymmetric weights (zeros: int16 [N, K/group]), any M: the
// tiled kernel with exact codes n - z and per-group fp32 scaling.
// The tiled kernel addresses a block's rows with 32-bit offsets; rows
// longer than kTiledMaxK elements run on the VALU path instead.
constexpr int64_t kTiledMaxK = (int64_t)1 << 22;
hipError_t launch_gemm_mfma_asym(const uint16_t* X, int64_t M, const uint32_t* packed,
                                 const uint16_t* scales, const int16_t* zeros, int64_t N,
                                 int64_t K, uint16_t* Y, hipStream_t stream, int num_cu,
                                 int gshift = 2);

// Prefill with K split over blocks (gemm_mfma.hip, symmetric weights): when
// the output has too few 128 x 256 block tiles to give most compute units a
// block (long-K shapes such as the FFN down projection), block (tile, z)
// takes the groups [z * groups_per_slice, ...) of K and stores its fp32
// partial tile to a workspace; a second kernel adds the slices of each tile
// in slice order and writes Y.
struct TiledSplit {
    int ksplit;              // K slices (1: no split)
    int groups_per_slice;
    int tiles;               // output tiles of bm x 256
    size_t workspace_bytes;  // tiles * ksplit * bm x 256 fp32 partials
    void* partials;          // filled in by the launcher
};
// The split used for (M, N, K) on num_cu compute units with bm x 256 tiles
// (128 symmetric, 64 asymmetric; ksplit == 1 when the shape is not split);
// ksplit > 0 forces a slice count, for measurements.
TiledSplit plan_tiled_split(int64_t M, int64_t N, int64_t K, int num_cu, int ksplit = 0,
                            int bm = 128);
// Requires plan.ksplit > 1 (a plan for bm = 128) and a workspace of
// plan.workspace_bytes.
hipError_t launch_gemm_tiled_split(const uint16_t* X, int64_t M, const uint32_t* packed,
                                   const uint16_t* scales, int64_t N, int64_t K, uint16_t* Y,
                                   hipStream_t stream, int gshift, const TiledSplit& plan,
                                   void* workspace);
// Asymmetric weights at group 128: a plan for bm = 64, 64 x 256 blocks.
hipError_t launch_gemm_tiled_split_asym(const uint16_t* X, int64_t M, const uint32_t* packed,
                                        const uint16_t* scales, const int16_t* zeros, int64_t N,
                                        int64_t K, uint16_t* Y, hipStream_t stream,
                                        const TiledSplit& plan, void* workspace);

// Activations in the act-order column order (gather_x.hip): Xp[m, j] =
// X[m, perm[j]], 0 for an index outside [0, K).  X, Xp fp16 [M, K] (16-byte
// aligned, not overlapping), perm device int32 [K] (16-byte aligned).
hipError_t launch_gather_x(const uint16_t* X, int64_t M, int64_t K, const int* perm,
                           uint16_t* Xp, hipStream_t stream, int num_cu);

// MFMA GEMV for M <= 4 with x resident in LDS (gemv_mfma4.hip): the weight
// stream of the VALU GEMV, products on v_mfma_f32_4x4x4_16b_f16.
constexpr int64_t kMfma4MaxM = 4;
// x of up to 152 KiB: with the row padding and the partial sums of two
// waves per row group the kernel's LDS stays below 160 KiB (M = 4 at K =
// 18944, the Qwen-2.5-7B down projection, fits).
constexpr int64_t kMfma4MaxXBytes = 152 * 1024;
hipError_t launch_gemv_mfma4(const uint16_t* X, int64_t M, const uint32_t* packed,
                             const uint16_t* scales, int64_t N, int64_t K, uint16_t* Y,
                             hipStream_t stream, int num_cu);

// MFMA path for batched decode, M <= 32 (gemm_batched.hip): blocks own
// contiguous weight rows, X staged through LDS in chunks of K.  Requires
// K <= kBatchedMaxK (32-bit buffer offsets).
constexpr int64_t kBatchedMaxM = 32;
constexpr int64_t kBatchedMaxK = (int64_t)1 << 24;
hipError_t launch_gemm_batched(const uint16_t* X, int64_t M, const uint32_t* packed,
                               const uint16_t* scales, int64_t N, int64_t K, uint16_t* Y,
                               hipStream_t stream, int num_cu);
// The same for asymmetric weights (zeros: int16 [N, K/128]).
hipError_t launch_gemm_batched_asym(const uint16_t* X, int64_t M, const uint32_t* packed,
                                    const uint16_t* scales, const int16_t* zeros, int64_t N,
                                    int64_t K, uint16_t* Y, hipStream_t stream, int num_cu);

// Batched decode with K split over blocks (gemm_batched.hip): block (b, k)
// owns rows_per_block rows and groups [k * groups_per_slice, ...) of K; the
// fp32 partial tiles go to a caller workspace (counters, then partials) and
// the last slice of each row block adds them in slice order.
constexpr int64_t kBatchedSplitCounters = 1024;   // row-block counters at the workspace start
struct BatchedSplit {
    int ksplit;              // K slices (1: no split)
    int groups_per_slice;
    int rows_per_block;
    int tile_rows;           // rows of the block's wave tiles (>= rows_per_block)
    int tile_m;              // 16 or 32 rows of X per tile
    size_t counter_bytes;    // kBatchedSplitCounters uint32, for every shape
    size_t workspace_bytes;  // counters + row blocks * slices * tile_rows * tile_m * 4
    uint32_t* counters;      // filled in by the launcher
    void* partials;
};
// The split used for (M, N, K) on num_cu compute units (rows, ksplit > 0
// force a shape, for measurements); ksplit == 1 when no split applies.
BatchedSplit plan_batched_split(int64_t M, int64_t N, int64_t K, int num_cu, int64_t rows = 0,
                                int ksplit = 0);
// Requires plan.ksplit > 1 and a workspace of plan.workspace_bytes whose
// counters are zero (every call leaves them zero).
hipError_t launch_gemm_batched_split(const uint16_t* X, int64_t M, const uint32_t* packed,
                                     const uint16_t* scales, int64_t N, int64_t K, uint16_t* Y,
                                     hipStream_t stream, const BatchedSplit& plan,
                                     void* workspace);

// MFMA path for few rows of X (gemm_skinny.hip): weights streamed once,
// waves split K.  Requires K <= kSkinnyMaxK (32-bit buffer offsets).
constexpr int64_t kSkinnyMaxK = (int64_t)1 << 24;
hipError_t launch_gemm_skinny(const uint16_t* X, int64_t M, const uint32_t* packed,
                              const uint16_t* scales, int64_t N, int64_t K, uint16_t* Y,
                              hipStream_t stream, int num_cu);

// Dependent sequence of M = 1 GEMVs in one launch (gemv_chain.hip).
constexpr int kChainMax = 64;           // stages per launch (kernel-argument size)
constexpr int kChainMaxK = 32768;       // x of a stage is held in LDS
constexpr int64_t kChainMaxN = (int64_t)1 << 20;
constexpr int kChainLineWords = 64;     // sync counters 256 bytes apart
constexpr int kChainLeaves = 8;         // first level of the arrival tree
constexpr int kChainErrWord = 0;
constexpr int kChainSyncWords = 1024;
static_assert((3 + kChainLeaves) * kChainLineWords <= kChainSyncWords, "sync layout");

struct ChainStageDev {
    const uint16_t* x;
    const uint32_t* packed;
    const uint16_t* scales;
    uint16_t* y;
    int N;
    int K;
};
struct ChainArgs {
    ChainStageDev st[kChainMax];
    int count;
    int x_vecs;          // LDS x capacity in 16-byte vectors (max K / 8)
    uint32_t* sync;
    // NULL: the error word stays set in `sync` (sticky).  Otherwise the last
    // block writes this call's error word here and clears it in `sync`.
    uint32_t* status;
};

// Launches one block per compute unit (co-resident); *blocks_out receives
// the grid size.  max_n: the largest N of the stages.
hipError_t launch_gemv_chain(const ChainArgs& args, int64_t max_n, hipStream_t stream,
                             int num_cu, int* blocks_out);

// The same with the counters in the library's own per-device array (fixed
// size kChainSyncWords words, zero when the library is loaded and after every
// call); args.sync is filled in here, args.status must be set.  `device` is
// the current HIP device.
hipError_t launch_gemv_chain_noalloc(ChainArgs& args, int64_t max_n, hipStream_t stream,
                                     int num_cu, int device);

}  // namespace w4a16

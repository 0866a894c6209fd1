// api.hip — the C ABI of include/w4a16.h: host-side validation, device
// checks and dispatch to the kernels.  The one device allocation is the
// copy of the activations in act-order column order that the matrix-core
// path of the act-order linear layer reads when the caller passes no
// workspace: stream-ordered, from a pool the library keeps per device.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string.h>

#include "w4a16.h"
#include "w4a16_launch.h"

namespace {

// Launch grids stay within the dispatch limits for M, N <= 2^24; kernels
// index K with int.
constexpr int64_t kMaxRows = (int64_t)1 << 24;
constexpr int64_t kMaxK = ((int64_t)1 << 31) - 128;

// Largest M sent to the VALU path by W4A16_ALGO_AUTO.
constexpr int64_t kValuMaxM = 2;

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// [p, p + bytes) and [q, q + qbytes) intersect (both non-empty).
bool overlap(const void* p, size_t bytes, const void* q, size_t qbytes) {
    if (bytes == 0 || qbytes == 0) return false;
    const uintptr_t a = (uintptr_t)p, b = (uintptr_t)q;
    return a < b + qbytes && b < a + bytes;
}

// Per-device facts, filled on first use of each device.
struct DeviceInfo {
    bool probed = false;
    bool ok = false;
    int num_cu = 0;
    hipMemPool_t pool = nullptr;   // stream-ordered scratch (act-order copies of X)
};
// Memory the pool keeps across synchronizations instead of returning it to
// the system (larger copies are returned after use).
constexpr uint64_t kPoolKeepBytes = (uint64_t)512 << 20;
constexpr int kMaxDevices = 64;
DeviceInfo g_devices[kMaxDevices];
std::mutex g_mutex;

int current_device(int* num_cu) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return W4A16_ERR_DEVICE;
    std::lock_guard<std::mutex> lock(g_mutex);
    DeviceInfo& d = g_devices[dev];
    if (!d.probed) {
        hipDeviceProp_t prop;
        d.probed = true;
        if (hipGetDeviceProperties(&prop, dev) == hipSuccess) {
            d.ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
            d.num_cu = prop.multiProcessorCount;
        }
    }
    if (!d.ok) return W4A16_ERR_DEVICE;
    *num_cu = d.num_cu;
    return W4A16_OK;
}

// The library's memory pool on the current device (created on first use).
hipMemPool_t device_pool() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_mutex);
    DeviceInfo& d = g_devices[dev];
    if (d.pool == nullptr) {
        hipMemPoolProps props;
        memset(&props, 0, sizeof(props));
        props.allocType = hipMemAllocationTypePinned;
        props.handleTypes = hipMemHandleTypeNone;
        props.location.type = hipMemLocationTypeDevice;
        props.location.id = dev;
        hipMemPool_t pool = nullptr;
        if (hipMemPoolCreate(&pool, &props) != hipSuccess) return nullptr;
        uint64_t keep = kPoolKeepBytes;
        (void)hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &keep);
        d.pool = pool;
    }
    return d.pool;
}

int check_sizes(int64_t M, int64_t N, int64_t K) {
    if (M < 0 || N < 0 || K < 0) return W4A16_ERR_INVALID_ARG;
    if (M > kMaxRows || N > kMaxRows || K > kMaxK) return W4A16_ERR_INVALID_ARG;
    if (K % W4A16_GROUP != 0) return W4A16_ERR_SHAPE;
    return W4A16_OK;
}

// Group sizes the kernels take: 32, 64, 128 or 256 elements per scale, and
// K a multiple of the group (K % 128 == 0 is required for every group); or
// W4A16_PER_CHANNEL, one scale per row.
int check_group(int64_t group, int64_t K) {
    if (group == W4A16_PER_CHANNEL) return W4A16_OK;
    if (group != 32 && group != 64 && group != 128 && group != 256) return W4A16_ERR_INVALID_ARG;
    if (K % group != 0) return W4A16_ERR_SHAPE;
    return W4A16_OK;
}

// log2(group / 32): the GEMV reads one scale per 2^gshift 32-code chunks.
int group_shift(int64_t group) {
    if (group == W4A16_PER_CHANNEL) return w4a16::kPerChannelShift;
    return group == 32 ? 0 : group == 64 ? 1 : group == 128 ? 2 : 3;
}

// Scales (and zero points) per row.
int64_t groups_per_row(int64_t K, int64_t group) {
    return group == W4A16_PER_CHANNEL ? (K > 0 ? 1 : 0) : K / group;
}

int status_of(hipError_t e) { return e == hipSuccess ? W4A16_OK : W4A16_ERR_LAUNCH; }

// The K split over blocks of the prefill kernel (w4a16_gemm_ws): symmetric
// weights, more than 64 rows, too few 128 x 256 output tiles for the compute
// units.  With K > N (long rows, few tiles) whenever the planner splits;
// with K <= N only where each slice holds at least 10 groups and the split
// grid still gives 3/4 of the compute units a block: there the unsplit
// kernel's smaller tiles do about as well (M = 128 / 256 / 512, us, unsplit
// against split: 4096x14336 M = 128 28.4 against 30.1 with 8 groups a slice,
// 4096x4096 21-28 against 25-31 on 64-128 blocks; split where taken:
// 3584x18944 M = 128 49.5 against 37.2, 8192x28672 M = 128 86.5 against
// 77.7-80.2, 4096x14336 M = 256 45.0 against 43.2-43.8).
w4a16::TiledSplit tiled_plan(int64_t M, int64_t N, int64_t K, int num_cu, bool asym) {
    w4a16::TiledSplit none{};
    none.ksplit = 1;
    if (asym) return none;
    const w4a16::TiledSplit p = w4a16::plan_tiled_split(M, N, K, num_cu);
    if (K > N || p.ksplit < 2) return p;
    const bool long_slices = p.groups_per_slice >= 10;
    const bool fills = (int64_t)p.tiles * p.ksplit * 4 >= (int64_t)num_cu * 3;
    return long_slices && fills ? p : none;
}

// The K split of asymmetric prefill (w4a16_gemm_asym_ws): group 128, more
// than 64 rows, K > N, 64 x 256 tiles in at least three slices.  With two
// slices (M = 512 on the FFN down projections) the split was as often slower
// as faster (18944x3584 138.6 against 126.6 us, 14336x4096 88.2 against
// 91.9); with three or more it gains (14336x4096 M = 128 / 256: 37.0 / 51.5
// against 72.3 / 70.8 us, 18944x3584 M = 128 70.7 against 99.6).
w4a16::TiledSplit asym_plan(int64_t M, int64_t N, int64_t K, int64_t group, int num_cu) {
    w4a16::TiledSplit none{};
    none.ksplit = 1;
    if (group != 128 || K <= N) return none;
    const w4a16::TiledSplit p = w4a16::plan_tiled_split(M, N, K, num_cu, 0, 64);
    return p.ksplit >= 3 ? p : none;
}

bool stream_capturing(hipStream_t s) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    return hipStreamIsCapturing(s, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone;
}

// perm: NULL, or the act-order column order (device int32 [K]).  zeros
// (asym): the int16 zero points of asymmetric weights, [N, K/group].
int linear(const uint16_t* X, int64_t M, const uint32_t* packed, const uint16_t* scales,
           int64_t N, int64_t K, int64_t group, uint16_t* Y, int algo, void* stream,
           const int32_t* perm = nullptr, bool with_perm = false,
           const int16_t* zeros = nullptr, bool asym = false, void* workspace = nullptr,
           size_t workspace_bytes = 0) {
    int st = check_sizes(M, N, K);
    if (st != W4A16_OK) return st;
    st = check_group(group, K);
    if (st != W4A16_OK) return st;
    if (algo != W4A16_ALGO_AUTO && algo != W4A16_ALGO_VALU && algo != W4A16_ALGO_MFMA)
        return W4A16_ERR_INVALID_ARG;
    if (M == 0 || N == 0) return W4A16_OK;
    // With K == 0 the inputs hold no bytes and may be NULL; they are never read.
    if (!Y || (K > 0 && (!X || !packed || !scales || (with_perm && !perm) || (asym && !zeros))))
        return W4A16_ERR_INVALID_ARG;
    if (!aligned(X, 16) || !aligned(packed, 16) || !aligned(scales, 2) || !aligned(Y, 2) ||
        !aligned(perm, 16) || !aligned(zeros, 2))
        return W4A16_ERR_MISALIGNED;
    const size_t y_bytes = (size_t)M * N * 2;
    const size_t s_bytes = (size_t)N * groups_per_row(K, group) * 2;
    if (overlap(Y, y_bytes, X, (size_t)M * K * 2) ||
        overlap(Y, y_bytes, packed, (size_t)N * K / 2) || overlap(Y, y_bytes, scales, s_bytes) ||
        (with_perm && overlap(Y, y_bytes, perm, (size_t)K * 4)) ||
        (asym && overlap(Y, y_bytes, zeros, s_bytes)))
        return W4A16_ERR_INVALID_ARG;
    // workspace (the act-order copy of X): 2 M K bytes, apart from every
    // operand
    const size_t xp_bytes = (size_t)M * K * 2;
    if (workspace != nullptr && with_perm && K > 0) {
        if (workspace_bytes < xp_bytes) return W4A16_ERR_INVALID_ARG;
        if (!aligned(workspace, 16)) return W4A16_ERR_MISALIGNED;
        if (overlap(workspace, xp_bytes, X, xp_bytes) || overlap(workspace, xp_bytes, Y, y_bytes) ||
            overlap(workspace, xp_bytes, packed, (size_t)N * K / 2) ||
            overlap(workspace, xp_bytes, scales, s_bytes) ||
            overlap(workspace, xp_bytes, perm, (size_t)K * 4) ||
            (asym && overlap(workspace, xp_bytes, zeros, s_bytes)))
            return W4A16_ERR_INVALID_ARG;
    }
    int num_cu = 0;
    st = current_device(&num_cu);
    if (st != W4A16_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    // Act order on the matrix cores needs a permuted copy of X: in the
    // caller's workspace, else allocated on the stream from the library's
    // pool; without a workspace a stream under graph capture keeps the VALU
    // path, which gathers x itself and allocates nothing.
    const bool capturing =
        with_perm && K > 0 && algo != W4A16_ALGO_VALU && workspace == nullptr &&
        stream_capturing(s);
    const bool valu = algo == W4A16_ALGO_VALU || (algo == W4A16_ALGO_AUTO && M <= kValuMaxM) ||
                      capturing;
    if (valu)
        return status_of(w4a16::launch_gemv_valu(X, M, packed, scales, N, K, Y, s, num_cu,
                                                 group_shift(group),
                                                 with_perm ? perm : nullptr,
                                                 asym ? zeros : nullptr));
    const uint16_t* Xm = X;
    void* xp = nullptr;       // pool memory to give back
    if (with_perm && K > 0) {
        void* dst = workspace;
        if (dst == nullptr) {
            hipMemPool_t pool = device_pool();
            if (pool == nullptr || hipMallocFromPoolAsync(&xp, xp_bytes, pool, s) != hipSuccess)
                return W4A16_ERR_LAUNCH;
            dst = xp;
        }
        const hipError_t e =
            w4a16::launch_gather_x(X, M, K, perm, static_cast<uint16_t*>(dst), s, num_cu);
        if (e != hipSuccess) {
            if (xp != nullptr) (void)hipFreeAsync(xp, s);
            return W4A16_ERR_LAUNCH;
        }
        Xm = static_cast<const uint16_t*>(dst);
    }
    const hipError_t e =
        asym ? w4a16::launch_gemm_mfma_asym(Xm, M, packed, scales, zeros, N, K, Y, s, num_cu,
                                            group_shift(group))
             : w4a16::launch_gemm_mfma(Xm, M, packed, scales, N, K, Y, s, num_cu,
                                       group_shift(group));
    if (xp != nullptr && hipFreeAsync(xp, s) != hipSuccess) return W4A16_ERR_LAUNCH;
    return status_of(e);
}

int quantize(const uint16_t* W, int64_t N, int64_t K, int64_t group, uint32_t* packed,
             uint16_t* scales, void* stream, const int32_t* perm = nullptr,
             bool with_perm = false, int16_t* zeros = nullptr, bool asym = false) {
    int st = check_sizes(0, N, K);
    if (st != W4A16_OK) return st;
    st = check_group(group, K);
    if (st != W4A16_OK) return st;
    if (N == 0 || K == 0) return W4A16_OK;
    if (!W || !packed || !scales || (with_perm && !perm) || (asym && !zeros))
        return W4A16_ERR_INVALID_ARG;
    if (!aligned(W, 16) || !aligned(packed, 16) || !aligned(scales, 2) || !aligned(perm, 16) ||
        !aligned(zeros, 2))
        return W4A16_ERR_MISALIGNED;
    const size_t w_bytes = (size_t)N * K * 2;
    const size_t p_bytes = (size_t)N * K / 2;
    const size_t s_bytes = (size_t)N * groups_per_row(K, group) * 2;
    const size_t perm_bytes = with_perm ? (size_t)K * 4 : 0;
    const size_t z_bytes = asym ? s_bytes : 0;
    // outputs: packed, scales, zeros; inputs: W, perm
    const void* outs[3] = {packed, scales, zeros};
    const size_t out_bytes[3] = {p_bytes, s_bytes, z_bytes};
    for (int i = 0; i < 3; ++i) {
        if (overlap(outs[i], out_bytes[i], W, w_bytes) ||
            overlap(outs[i], out_bytes[i], perm, perm_bytes))
            return W4A16_ERR_INVALID_ARG;
        for (int j = i + 1; j < 3; ++j)
            if (overlap(outs[i], out_bytes[i], outs[j], out_bytes[j])) return W4A16_ERR_INVALID_ARG;
    }
    int num_cu = 0;
    st = current_device(&num_cu);
    if (st != W4A16_OK) return st;
    return status_of(w4a16::launch_quantize(W, N, K, group, packed, scales,
                                            static_cast<hipStream_t>(stream), num_cu,
                                            with_perm ? perm : nullptr, asym ? zeros : nullptr));
}

// Q4_0 buffer: N rows of K/32 blocks of 18 bytes, rounded up to 16 bytes.
size_t q4_0_bytes(int64_t N, int64_t K) {
    return ((size_t)N * (size_t)(K / 32) * 18 + 15) & ~(size_t)15;
}

int linear_q4_0(const uint16_t* X, int64_t M, const uint8_t* blocks, int64_t N, int64_t K,
                uint16_t* Y, void* stream) {
    int st = check_sizes(M, N, K);
    if (st != W4A16_OK) return st;
    if (K > w4a16::kQ40MaxK) return W4A16_ERR_INVALID_ARG;
    if (M == 0 || N == 0) return W4A16_OK;
    if (!Y || (K > 0 && (!X || !blocks))) return W4A16_ERR_INVALID_ARG;
    if (!aligned(X, 16) || !aligned(blocks, 16) || !aligned(Y, 2)) return W4A16_ERR_MISALIGNED;
    const size_t y_bytes = (size_t)M * N * 2;
    if (overlap(Y, y_bytes, X, (size_t)M * K * 2) || overlap(Y, y_bytes, blocks, q4_0_bytes(N, K)))
        return W4A16_ERR_INVALID_ARG;
    int num_cu = 0;
    st = current_device(&num_cu);
    if (st != W4A16_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    // K == 0: the split-layout kernel writes the zeros (it reads no weights)
    if (K == 0)
        return status_of(w4a16::launch_gemv_valu(X, M, nullptr, nullptr, N, 0, Y, s, num_cu));
    return status_of(w4a16::launch_gemv_q4_0(X, M, blocks, N, K, Y, s, num_cu));
}

}  // namespace

extern "C" {

size_t w4a16_q4_0_bytes(int64_t N, int64_t K) {
    if (check_sizes(0, N, K) != W4A16_OK) return 0;
    return q4_0_bytes(N, K);
}

int w4a16_quantize_q4_0(const uint16_t* W, int64_t N, int64_t K, uint8_t* blocks, void* stream) {
    int st = check_sizes(0, N, K);
    if (st != W4A16_OK) return st;
    if (N == 0 || K == 0) return W4A16_OK;
    if (!W || !blocks) return W4A16_ERR_INVALID_ARG;
    if (!aligned(W, 16) || !aligned(blocks, 16)) return W4A16_ERR_MISALIGNED;
    if (overlap(blocks, q4_0_bytes(N, K), W, (size_t)N * K * 2)) return W4A16_ERR_INVALID_ARG;
    int num_cu = 0;
    st = current_device(&num_cu);
    if (st != W4A16_OK) return st;
    return status_of(w4a16::launch_quantize_q4_0(W, N, K, blocks, static_cast<hipStream_t>(stream)));
}

int w4a16_gemv_q4_0(const uint16_t* x, const uint8_t* blocks, int64_t N, int64_t K, uint16_t* y,
                    void* stream) {
    return linear_q4_0(x, 1, blocks, N, K, y, stream);
}

int w4a16_gemm_q4_0(const uint16_t* X, int64_t M, const uint8_t* blocks, int64_t N, int64_t K,
                    uint16_t* Y, void* stream) {
    return linear_q4_0(X, M, blocks, N, K, Y, stream);
}


size_t w4a16_packed_bytes(int64_t N, int64_t K) {
    if (check_sizes(0, N, K) != W4A16_OK) return 0;
    return (size_t)N * (size_t)K / 2;
}

size_t w4a16_scales_bytes(int64_t N, int64_t K) {
    return w4a16_scales_bytes_g(N, K, W4A16_GROUP);
}

size_t w4a16_scales_bytes_g(int64_t N, int64_t K, int64_t group) {
    if (check_sizes(0, N, K) != W4A16_OK || check_group(group, K) != W4A16_OK) return 0;
    return (size_t)N * (size_t)groups_per_row(K, group) * 2;
}

int w4a16_quantize(const uint16_t* W, int64_t N, int64_t K, uint32_t* packed, uint16_t* scales,
                   void* stream) {
    return quantize(W, N, K, W4A16_GROUP, packed, scales, stream);
}

int w4a16_quantize_g(const uint16_t* W, int64_t N, int64_t K, int64_t group, uint32_t* packed,
                     uint16_t* scales, void* stream) {
    return quantize(W, N, K, group, packed, scales, stream);
}

int w4a16_gemv(const uint16_t* x, const uint32_t* packed, const uint16_t* scales, int64_t N,
               int64_t K, uint16_t* y, void* stream) {
    return linear(x, 1, packed, scales, N, K, W4A16_GROUP, y, W4A16_ALGO_VALU, stream);
}

int w4a16_gemv_g(const uint16_t* x, const uint32_t* packed, const uint16_t* scales, int64_t N,
                 int64_t K, int64_t group, uint16_t* y, void* stream) {
    return linear(x, 1, packed, scales, N, K, group, y, W4A16_ALGO_VALU, stream);
}

int w4a16_gemm(const uint16_t* X, int64_t M, const uint32_t* packed, const uint16_t* scales,
               int64_t N, int64_t K, uint16_t* Y, void* stream) {
    return linear(X, M, packed, scales, N, K, W4A16_GROUP, Y, W4A16_ALGO_AUTO, stream);
}

int w4a16_gemm_g(const uint16_t* X, int64_t M, const uint32_t* packed, const uint16_t* scales,
                 int64_t N, int64_t K, int64_t group, uint16_t* Y, void* stream) {
    return linear(X, M, packed, scales, N, K, group, Y, W4A16_ALGO_AUTO, stream);
}

int w4a16_gemm_ex(const uint16_t* X, int64_t M, const uint32_t* packed, const uint16_t* scales,
                  int64_t N, int64_t K, uint16_t* Y, int algo, void* stream) {
    return linear(X, M, packed, scales, N, K, W4A16_GROUP, Y, algo, stream);
}

size_t w4a16_linear_workspace_bytes(int64_t M, int64_t K, int has_perm) {
    if (!has_perm || check_sizes(M, 0, K) != W4A16_OK) return 0;
    return (size_t)M * (size_t)K * 2;
}

int w4a16_linear(const uint16_t* X, int64_t M, const int32_t* perm, const uint32_t* packed,
                 const uint16_t* scales, const int16_t* zeros, int64_t N, int64_t K,
                 int64_t group, uint16_t* Y, int algo, void* workspace, size_t workspace_bytes,
                 void* stream) {
    return linear(X, M, packed, scales, N, K, group, Y, algo, stream, perm, perm != nullptr,
                  zeros, zeros != nullptr, workspace, workspace_bytes);
}

}  // extern "C"

namespace {

// The K-split plan w4a16_gemm_ws uses: the batched-decode shapes that the
// automatic choice sends to the batched matrix-core kernel (above the 4x4x4
// GEMV's rows, at most 32 rows), when the planner splits them.
w4a16::BatchedSplit ws_plan(int64_t M, int64_t N, int64_t K, int num_cu) {
    w4a16::BatchedSplit none{};
    none.ksplit = 1;
    const bool batched = M > kValuMaxM && M <= w4a16::kBatchedMaxM && K > 0 &&
                         !(M <= w4a16::kMfma4MaxM && M * K * 2 <= w4a16::kMfma4MaxXBytes);
    return batched ? w4a16::plan_batched_split(M, N, K, num_cu) : none;
}

}  // namespace

extern "C" {

size_t w4a16_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (check_sizes(M, N, K) != W4A16_OK || M == 0 || N == 0) return 0;
    int num_cu = 0;
    if (current_device(&num_cu) != W4A16_OK) return 0;
    const w4a16::BatchedSplit p = ws_plan(M, N, K, num_cu);
    if (p.ksplit > 1) return p.workspace_bytes;
    const w4a16::TiledSplit t = tiled_plan(M, N, K, num_cu, false);
    return t.ksplit > 1 ? t.workspace_bytes : 0;
}

int w4a16_gemm_ws(const uint16_t* X, int64_t M, const uint32_t* packed, const uint16_t* scales,
                  int64_t N, int64_t K, uint16_t* Y, void* workspace, size_t workspace_bytes,
                  void* stream) {
    int st = check_sizes(M, N, K);
    if (st != W4A16_OK) return st;
    if (M == 0 || N == 0) return W4A16_OK;
    int num_cu = 0;
    // shapes the planner does not split run as w4a16_gemm (workspace unused)
    if (K > 0 && (!X || !packed || !scales || !Y)) return W4A16_ERR_INVALID_ARG;
    st = current_device(&num_cu);
    if (st != W4A16_OK) return st;
    const w4a16::BatchedSplit plan = ws_plan(M, N, K, num_cu);
    const w4a16::TiledSplit tplan = tiled_plan(M, N, K, num_cu, false);
    if (plan.ksplit < 2 && tplan.ksplit < 2) return w4a16_gemm(X, M, packed, scales, N, K, Y, stream);
    const size_t need = plan.ksplit > 1 ? plan.workspace_bytes : tplan.workspace_bytes;
    if (!workspace || workspace_bytes < need) return W4A16_ERR_INVALID_ARG;
    if (!aligned(X, 16) || !aligned(packed, 16) || !aligned(scales, 2) || !aligned(Y, 2) ||
        !aligned(workspace, 256))
        return W4A16_ERR_MISALIGNED;
    const size_t y_bytes = (size_t)M * N * 2, x_bytes = (size_t)M * K * 2;
    const size_t p_bytes = (size_t)N * K / 2, s_bytes = (size_t)N * (K / W4A16_GROUP) * 2;
    const size_t w_bytes = need;
    if (overlap(Y, y_bytes, X, x_bytes) || overlap(Y, y_bytes, packed, p_bytes) ||
        overlap(Y, y_bytes, scales, s_bytes) || overlap(workspace, w_bytes, X, x_bytes) ||
        overlap(workspace, w_bytes, Y, y_bytes) || overlap(workspace, w_bytes, packed, p_bytes) ||
        overlap(workspace, w_bytes, scales, s_bytes))
        return W4A16_ERR_INVALID_ARG;
    if (plan.ksplit < 2)
        return status_of(w4a16::launch_gemm_tiled_split(X, M, packed, scales, N, K, Y,
                                                        static_cast<hipStream_t>(stream), 2, tplan,
                                                        workspace));
    return status_of(w4a16::launch_gemm_batched_split(X, M, packed, scales, N, K, Y,
                                                      static_cast<hipStream_t>(stream), plan,
                                                      workspace));
}

size_t w4a16_gemm_asym_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t group) {
    if (check_sizes(M, N, K) != W4A16_OK || check_group(group, K) != W4A16_OK) return 0;
    int num_cu = 0;
    if (current_device(&num_cu) != W4A16_OK) return 0;
    const w4a16::TiledSplit p = asym_plan(M, N, K, group, num_cu);
    return p.ksplit > 1 ? p.workspace_bytes : 0;
}

int w4a16_gemm_asym_ws(const uint16_t* X, int64_t M, const uint32_t* packed,
                       const uint16_t* scales, const int16_t* zeros, int64_t N, int64_t K,
                       int64_t group, uint16_t* Y, void* workspace, size_t workspace_bytes,
                       void* stream) {
    int st = check_sizes(M, N, K);
    if (st != W4A16_OK) return st;
    st = check_group(group, K);
    if (st != W4A16_OK) return st;
    if (M == 0 || N == 0) return W4A16_OK;
    if (K > 0 && (!X || !packed || !scales || !zeros || !Y)) return W4A16_ERR_INVALID_ARG;
    int num_cu = 0;
    st = current_device(&num_cu);
    if (st != W4A16_OK) return st;
    const w4a16::TiledSplit plan = asym_plan(M, N, K, group, num_cu);
    // shapes the planner does not split run as w4a16_gemm_asym (workspace unused)
    if (plan.ksplit < 2)
        return w4a16_gemm_asym(X, M, nullptr, packed, scales, zeros, N, K, group, Y, stream);
    if (!workspace || workspace_bytes < plan.workspace_bytes) return W4A16_ERR_INVALID_ARG;
    if (!aligned(X, 16) || !aligned(packed, 16) || !aligned(scales, 2) || !aligned(zeros, 2) ||
        !aligned(Y, 2) || !aligned(workspace, 256))
        return W4A16_ERR_MISALIGNED;
    const size_t y_bytes = (size_t)M * N * 2, x_bytes = (size_t)M * K * 2;
    const size_t p_bytes = (size_t)N * K / 2, s_bytes = (size_t)N * (K / group) * 2;
    const size_t w_bytes = plan.workspace_bytes;
    if (overlap(Y, y_bytes, X, x_bytes) || overlap(Y, y_bytes, packed, p_bytes) ||
        overlap(Y, y_bytes, scales, s_bytes) || overlap(Y, y_bytes, zeros, s_bytes) ||
        overlap(workspace, w_bytes, X, x_bytes) || overlap(workspace, w_bytes, Y, y_bytes) ||
        overlap(workspace, w_bytes, packed, p_bytes) ||
        overlap(workspace, w_bytes, scales, s_bytes) ||
        overlap(workspace, w_bytes, zeros, s_bytes))
        return W4A16_ERR_INVALID_ARG;
    return status_of(w4a16::launch_gemm_tiled_split_asym(X, M, packed, scales, zeros, N, K, Y,
                                                         static_cast<hipStream_t>(stream), plan,
                                                         workspace));
}

int w4a16_quantize_perm(const uint16_t* W, const int32_t* perm, int64_t N, int64_t K,
                        uint32_t* packed, uint16_t* scales, void* stream) {
    return quantize(W, N, K, W4A16_GROUP, packed, scales, stream, perm, true);
}

int w4a16_gemv_perm(const uint16_t* x, const int32_t* perm, const uint32_t* packed,
                    const uint16_t* scales, int64_t N, int64_t K, uint16_t* y, void* stream) {
    return linear(x, 1, packed, scales, N, K, W4A16_GROUP, y, W4A16_ALGO_VALU, stream, perm,
                  true);
}

int w4a16_gemm_perm(const uint16_t* X, int64_t M, const int32_t* perm, const uint32_t* packed,
                    const uint16_t* scales, int64_t N, int64_t K, uint16_t* Y, void* stream) {
    return linear(X, M, packed, scales, N, K, W4A16_GROUP, Y, W4A16_ALGO_AUTO, stream, perm,
                  true);
}

int w4a16_quantize_asym(const uint16_t* W, const int32_t* perm, int64_t N, int64_t K,
                        int64_t group, uint32_t* packed, uint16_t* scales, int16_t* zeros,
                        void* stream) {
    return quantize(W, N, K, group, packed, scales, stream, perm, perm != nullptr, zeros, true);
}

int w4a16_gemv_asym(const uint16_t* x, const int32_t* perm, const uint32_t* packed,
                    const uint16_t* scales, const int16_t* zeros, int64_t N, int64_t K,
                    int64_t group, uint16_t* y, void* stream) {
    return linear(x, 1, packed, scales, N, K, group, y, W4A16_ALGO_VALU, stream, perm,
                  perm != nullptr, zeros, true);
}

int w4a16_gemm_asym(const uint16_t* X, int64_t M, const int32_t* perm, const uint32_t* packed,
                    const uint16_t* scales, const int16_t* zeros, int64_t N, int64_t K,
                    int64_t group, uint16_t* Y, void* stream) {
    return linear(X, M, packed, scales, N, K, group, Y, W4A16_ALGO_AUTO, stream, perm,
                  perm != nullptr, zeros, true);
}

}  // extern "C"

namespace {

// Validates a chain of stages and fills `args`.  `extra`, `extra_bytes`: a
// caller buffer the chain writes (the sync buffer or the status word) that
// must not overlap any stage's tensors; NULL for none.
int chain_args(const w4a16_gemv_stage* stages, int count, const void* extra, size_t extra_bytes,
               w4a16::ChainArgs* args, int64_t* max_n_out) {
    static_assert(W4A16_CHAIN_MAX == w4a16::kChainMax, "chain limit");
    static_assert(W4A16_CHAIN_SYNC_WORDS == w4a16::kChainSyncWords, "sync words");
    static_assert(W4A16_CHAIN_ERR_WORD == w4a16::kChainErrWord, "error word");
    if (!stages) return W4A16_ERR_INVALID_ARG;
    memset(args, 0, sizeof(*args));
    int64_t max_k = 0, max_n = 0;
    for (int s = 0; s < count; ++s) {
        const w4a16_gemv_stage& st = stages[s];
        if (st.N < 1 || st.N > w4a16::kChainMaxN || st.K < 0 || st.K > w4a16::kChainMaxK)
            return W4A16_ERR_INVALID_ARG;
        if (st.K % W4A16_GROUP != 0 || st.K == 0) return W4A16_ERR_SHAPE;
        if (!st.x || !st.packed || !st.scales || !st.y) return W4A16_ERR_INVALID_ARG;
        if (!aligned(st.x, 16) || !aligned(st.packed, 16) || !aligned(st.scales, 2) ||
            !aligned(st.y, 2))
            return W4A16_ERR_MISALIGNED;
        if (st.K > max_k) max_k = st.K;
        if (st.N > max_n) max_n = st.N;
    }
    for (int s = 0; s < count; ++s) {
        const w4a16_gemv_stage& a = stages[s];
        const size_t yb = (size_t)a.N * 2;
        if (overlap(a.y, yb, a.x, (size_t)a.K * 2) || overlap(a.y, yb, extra, extra_bytes) ||
            overlap(a.x, (size_t)a.K * 2, extra, extra_bytes))
            return W4A16_ERR_INVALID_ARG;
        for (int t = 0; t < count; ++t) {
            const w4a16_gemv_stage& b = stages[t];
            // Stages run in order, so outputs may alias each other and later
            // inputs; weights are prefetched across stages, so no output may
            // alias any stage's weights.
            if (overlap(a.y, yb, b.packed, (size_t)b.N * b.K / 2) ||
                overlap(a.y, yb, b.scales, (size_t)b.N * (b.K / W4A16_GROUP) * 2))
                return W4A16_ERR_INVALID_ARG;
            if (overlap(extra, extra_bytes, b.packed, (size_t)b.N * b.K / 2) ||
                overlap(extra, extra_bytes, b.scales, (size_t)b.N * (b.K / W4A16_GROUP) * 2))
                return W4A16_ERR_INVALID_ARG;
        }
        args->st[s] = w4a16::ChainStageDev{a.x, a.packed, a.scales, a.y, (int)a.N, (int)a.K};
    }
    args->count = count;
    args->x_vecs = (int)(max_k / 8);
    *max_n_out = max_n;
    return W4A16_OK;
}

}  // namespace

extern "C" {

int w4a16_gemv_chain(const w4a16_gemv_stage* stages, int count, uint32_t* sync, void* stream) {
    if (count < 0 || count > W4A16_CHAIN_MAX) return W4A16_ERR_INVALID_ARG;
    if (count == 0) return W4A16_OK;
    if (!sync) return W4A16_ERR_INVALID_ARG;
    if (!aligned(sync, 4)) return W4A16_ERR_MISALIGNED;
    w4a16::ChainArgs args;
    int64_t max_n = 0;
    int st = chain_args(stages, count, sync, (size_t)W4A16_CHAIN_SYNC_WORDS * 4, &args, &max_n);
    if (st != W4A16_OK) return st;
    args.sync = sync;
    int num_cu = 0;
    st = current_device(&num_cu);
    if (st != W4A16_OK) return st;
    int blocks = 0;
    return status_of(w4a16::launch_gemv_chain(args, max_n, static_cast<hipStream_t>(stream),
                                              num_cu, &blocks));
}

int w4a16_gemv_chain_noalloc(const w4a16_gemv_stage* stages, int count, uint32_t* status,
                             void* stream) {
    if (count < 0 || count > W4A16_CHAIN_MAX) return W4A16_ERR_INVALID_ARG;
    if (count == 0) return W4A16_OK;
    if (!status) return W4A16_ERR_INVALID_ARG;
    if (!aligned(status, 4)) return W4A16_ERR_MISALIGNED;
    w4a16::ChainArgs args;
    int64_t max_n = 0;
    int st = chain_args(stages, count, status, 4, &args, &max_n);
    if (st != W4A16_OK) return st;
    args.status = status;
    int num_cu = 0;
    st = current_device(&num_cu);
    if (st != W4A16_OK) return st;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return W4A16_ERR_DEVICE;
    return status_of(w4a16::launch_gemv_chain_noalloc(args, max_n,
                                                      static_cast<hipStream_t>(stream), num_cu,
                                                      dev));
}

int64_t w4a16_valu_max_m(void) { return kValuMaxM; }

const char* w4a16_status_string(int status) {
    switch (status) {
        case W4A16_OK: return "ok";
        case W4A16_ERR_INVALID_ARG: return "invalid argument (null pointer, negative or too large size, overlapping output, unknown algo or group size)";
        case W4A16_ERR_SHAPE: return "K must be a multiple of 128 and of the group size";
        case W4A16_ERR_MISALIGNED: return "misaligned pointer (W, X, x, packed, perm need 16 bytes; scales, zeros, Y, y need 2)";
        case W4A16_ERR_DEVICE: return "no HIP device, or the current device is not gfx950";
        case W4A16_ERR_LAUNCH: return "the HIP runtime rejected a kernel launch";
        default: return "unknown status";
    }
}

}  // extern "C"

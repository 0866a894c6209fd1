/*
 * w4a16.h — C ABI of the W4A16 linear layer for AMD Instinct MI355X (gfx950).
 *
 * Weight-only INT4: fp16 weights W[N,K] (N = out_features, K = in_features)
 * are quantized round-to-nearest, symmetric, one fp16 scale per group of 128
 * consecutive elements along K; activations stay fp16 and the weights are
 * dequantized in registers inside the GEMV/GEMM kernels.
 *
 * Sources (web pages; cited by key in every comment of this library):
 *   [BENCH] "W4A16 量化算子解码性能基准跑分与端侧大模型推理显存实测报告"
 *           (W4A16 operator decode benchmark report), mhpq.cn/news/1206820.
 *           §一 test setup (group 128, symmetric INT4, fp16 scales),
 *           §二 results (decode is memory-bound, every token sweeps all
 *           weights), §五 lessons (dequantize on the fly in registers).
 *   [QUANT] qaqbuyan.com article 126 on LLM quantization, section
 *           "量化的数学基石——从 IEEE 754 到量化误差":
 *           sub-section 1 (FP16 bit layout, INT4 range [-8,7]),
 *           sub-section 2 (symmetric quantization equations; rounding error
 *           uniform in [-s/2, s/2]),
 *           sub-section 3 (granularity table; per-group quantizer listing
 *           with group 128 along in_features, two nibbles per byte, offset
 *           binary q+8, even index in the low nibble; 3.1% scale overhead).
 *   [INT4]  guijiagi.com tag page "量化", entry on INT8 / INT4 / FP8
 *           schemes, "INT4量化" paragraph and its group-quantization example.
 *
 * Packed layout (one row n of W; word j of the row holds elements 8j..8j+7):
 *     packed[n*(K/8) + j] = sum_{i=0..7} ((q[n][8j+i] + 8) & 0xF) << (4*i)
 *     scales[n*(K/128) + g] = fp16 bits of s[n][g]
 * Read as little-endian bytes this is exactly the two-nibbles-per-byte,
 * even-index-low layout of [QUANT] sub-section 3's listing, widened to
 * eight nibbles per uint32.  Packed bytes: N*K/2; scale bytes: N*K/64.
 *
 * Quantizer, per row n and group g (k in [128g, 128g+128)):
 *     a = max_k |W[n,k]|
 *     s = round-to-nearest-even fp16 of a/7              ([QUANT] sub-sec. 2)
 *     q = clamp(round_half_even(W[n,k] / s), -8, 7)      ([QUANT] sub-sec. 2)
 *     q = 0 for every element when s == 0 (all-zero or underflowing group)
 * The quotient W/s is decided exactly (as with real numbers) and q is taken
 * against the stored fp16 scale, the only scale the dequantizer sees.
 *
 * Linear layer: Y[m,n] = sum_k X[m,k] * s[n,k/128] * q[n,k]  (Y = X·Ŵᵀ),
 * accumulated in fp32, written as fp16 (round to nearest even).
 *
 * Conventions shared by every entry point:
 *   - Every tensor pointer is a DEVICE pointer into memory the caller owns;
 *     the library allocates nothing and keeps no per-call state.
 *   - fp16 values are passed as their IEEE binary16 bit patterns (uint16_t).
 *   - All tensors are dense row-major with no padding between rows.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Work is enqueued
 *     asynchronously; nothing synchronizes.  Faults surface at the caller's
 *     next synchronization, as for any HIP launch.
 *   - Arguments are validated on the host before anything is enqueued; a
 *     non-zero status means nothing was enqueued.
 *   - Sizes: 0 <= M, N <= 2^24, 0 <= K < 2^31, K % 128 == 0.  M == 0 or
 *     N == 0 enqueues nothing (pointers may then be NULL).  K == 0 makes
 *     every output 0 (the inputs, which then hold no bytes, may be NULL).
 *   - Alignment: W, X, x and packed must be 16-byte aligned; scales, Y and
 *     y 2-byte aligned.
 *   - Outputs must not overlap any input.
 *   - Inputs must be finite (a precondition, not checked).
 *   - The current HIP device must be gfx950.
 */
#ifndef W4A16_H
#define W4A16_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define W4A16_GROUP 128

typedef enum {
    W4A16_OK = 0,
    W4A16_ERR_INVALID_ARG = 1, /* NULL pointer, negative size, size overflow, overlapping output */
    W4A16_ERR_SHAPE = 2,       /* K % 128 != 0, or K not a multiple of the group */
    W4A16_ERR_MISALIGNED = 3,  /* alignment rule above violated */
    W4A16_ERR_DEVICE = 4,      /* no HIP device, or the current device is not gfx950 */
    W4A16_ERR_LAUNCH = 5       /* the HIP runtime rejected a launch */
} w4a16_status;

enum {
    W4A16_ALGO_AUTO = 0, /* pick by M: VALU GEMV for small M, MFMA GEMM above the crossover */
    W4A16_ALGO_VALU = 1, /* force the VALU (dot-product) path, any M */
    W4A16_ALGO_MFMA = 2  /* force the MFMA path, any M */
};

/* Byte sizes of the packed weights (N*K/2) and the scales (N*(K/128)*2):
 * [QUANT] sub-section 3's per-group listing stores two 4-bit codes per byte
 * and one fp16 scale per group of 128 along in_features (its 3.1 % scale
 * overhead is 2 bytes per 64 code bytes).
 * Return 0 for negative sizes, K % 128 != 0 or overflow. */
size_t w4a16_packed_bytes(int64_t N, int64_t K);
size_t w4a16_scales_bytes(int64_t N, int64_t K);

/* Quantize and pack W ([QUANT] sub-sections 2-3; [INT4]).
 *   W       in : fp16 [N, K]
 *   packed  out: uint32 [N, K/8]   (layout above)
 *   scales  out: fp16 [N, K/128]
 * Bit-exact: exactly one correct output exists for every finite W. */
int w4a16_quantize(const uint16_t* W, int64_t N, int64_t K,
                   uint32_t* packed, uint16_t* scales, void* stream);

/* Decode GEMV, M = 1 ([BENCH] §二, §五):  y[n] = sum_k x[k] * ŵ[n,k].
 *   x       in : fp16 [K]
 *   packed  in : uint32 [N, K/8];  scales in : fp16 [N, K/128]
 *   y       out: fp16 [N] */
int w4a16_gemv(const uint16_t* x, const uint32_t* packed, const uint16_t* scales,
               int64_t N, int64_t K, uint16_t* y, void* stream);

/* Batched decode / prefill ([BENCH] §一 prompt of 512 tokens, §二 prefill):
 *   X in : fp16 [M, K];  Y out: fp16 [M, N];  Y = X·Ŵᵀ.
 * Picks the kernel by M (W4A16_ALGO_AUTO).
 * Accuracy (every entry point of the linear layer): fp32 accumulation, y
 * rounded to fp16 (RNE); |y - y_exact| <= 1e-3 sum_k |x_k ŵ_k| +
 * max(2^-10 |y_exact|, 2^-24) per element.  The matrix-core kernels that
 * multiply fp16 weights fp16(s*q) clamp them to +-65504 (only a group whose
 * absmax is 65504 reaches 7*s = 65520), within that bound; an output whose
 * exact value exceeds the fp16 range is +-infinity. */
int w4a16_gemm(const uint16_t* X, int64_t M, const uint32_t* packed, const uint16_t* scales,
               int64_t N, int64_t K, uint16_t* Y, void* stream);

/* w4a16_gemm with the kernel family forced by `algo` (W4A16_ALGO_*); an
 * unknown algo is W4A16_ERR_INVALID_ARG.  Results of every algo meet the same
 * tolerance; used to measure the VALU/MFMA crossover.  The operation is
 * w4a16_gemm's ([BENCH] §二: decode at one token, prefill at 512); only the
 * kernel family that computes it is chosen here. */
int w4a16_gemm_ex(const uint16_t* X, int64_t M, const uint32_t* packed, const uint16_t* scales,
                  int64_t N, int64_t K, uint16_t* Y, int algo, void* stream);

/* ---- Batched decode with K split over blocks ([BENCH] §二: decode of a few
 * tokens is one pass over the weights; the FFN down projection has K = 3.5 N,
 * so one block per compute unit would own 16 of its rows and read all of X
 * for them).  w4a16_gemm with a caller workspace: for the shapes that
 * w4a16_gemm_workspace_bytes reports a non-zero size for, blocks own more
 * rows and one slice of K each, store fp32 partial tiles in the workspace,
 * and the last slice of each row block to finish adds them in slice order
 * (deterministic) and writes Y.  Prefill ([BENCH] §一/§二, 512-token prompt)
 * with more than 64 rows and too few 128 x 256 output tiles for the compute
 * units (K > N; with K <= N where slices of at least 10 groups of K still
 * give 3/4 of the compute units a block) splits K over blocks too, with
 * 128 x 256 partial tiles, which a second kernel on the same stream adds in
 * slice order
 * (w4a16_gemm keeps these shapes unsplit, so that it never needs memory of
 * its own).  Other shapes run exactly as w4a16_gemm and
 * ignore the workspace.  Same accuracy
 * bound as w4a16_gemm; the sum order of split shapes differs, so their
 * results are not bit-identical to the unsplit kernel's.
 *   workspace  DEVICE, 256-byte aligned, at least
 *              w4a16_gemm_workspace_bytes(M, N, K) bytes, owned by the caller,
 *              all zero before its first use; every call leaves its counters
 *              zero again, so it is reused without clearing.  Calls sharing a
 *              workspace must not overlap in time (stream-ordered calls and
 *              graph replays are fine).  It must not overlap X, Y or the
 *              weights.
 * w4a16_gemm_workspace_bytes returns 0 for shapes that do not split, for
 * invalid sizes and when the current device is not gfx950 (the split depends
 * on the compute-unit count).  A workspace smaller than required is
 * W4A16_ERR_INVALID_ARG. */
size_t w4a16_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);
int w4a16_gemm_ws(const uint16_t* X, int64_t M, const uint32_t* packed, const uint16_t* scales,
                  int64_t N, int64_t K, uint16_t* Y, void* workspace, size_t workspace_bytes,
                  void* stream);

/* ---- Group size as a parameter ([QUANT] sub-section 3 granularity table:
 * group 128 is the default, group 32 for outlier-sensitive layers, per
 * channel one scale per output row; [QUANT] GPTQ section, group_size table:
 * 256, 128, 64 and 32 trade scale storage, 1.6 % to 12.5 %, against
 * accuracy, and -1 is per channel).  Same quantizer, layout and linear layer
 * as above with `group` elements per scale along K:
 *     scales[n*(K/group) + g] = fp16 bits of s[n][g],  g = k / group
 *     Y[m,n] = sum_k X[m,k] * s[n,k/group] * q[n,k]
 * group must be 32, 64, 128, 256 or W4A16_PER_CHANNEL (else
 * W4A16_ERR_INVALID_ARG) and divide K (else W4A16_ERR_SHAPE); K % 128 == 0
 * as everywhere.  W4A16_PER_CHANNEL is the group of the whole row (K
 * elements): one scale per row, scales[n], absmax over the row.  group ==
 * 128 gives exactly the functions above.  Scales bytes: N*(K/group)*2, N*2
 * per channel (0 for bad arguments).  w4a16_gemm_g picks the kernel by M
 * as w4a16_gemm does (the matrix cores above w4a16_valu_max_m(); for groups
 * other than 128 the tiled matrix-core kernel, whose 128-element K steps
 * read one scale per 32-element chunk of a lane). */
#define W4A16_PER_CHANNEL (-1)
size_t w4a16_scales_bytes_g(int64_t N, int64_t K, int64_t group);
int w4a16_quantize_g(const uint16_t* W, int64_t N, int64_t K, int64_t group,
                     uint32_t* packed, uint16_t* scales, void* stream);
int w4a16_gemv_g(const uint16_t* x, const uint32_t* packed, const uint16_t* scales,
                 int64_t N, int64_t K, int64_t group, uint16_t* y, void* stream);
int w4a16_gemm_g(const uint16_t* X, int64_t M, const uint32_t* packed, const uint16_t* scales,
                 int64_t N, int64_t K, int64_t group, uint16_t* Y, void* stream);

/* ---- Act-order column order ([QUANT] GPTQ section, act_order: columns are
 * quantized in an order perm (by Hessian diagonal) and, for inference, the
 * weight is kept in that order and the activations are permuted the same
 * way).  perm is a DEVICE int32 [K], 16-byte aligned; column j of the stored
 * weight is column perm[j] of W, groups of 128 are taken along the stored
 * order, and an index outside [0, K) reads as 0 (W or x).
 *   w4a16_quantize_perm:  packed/scales of W[:, perm]   (same as
 *                         w4a16_quantize on the column-permuted W)
 *   w4a16_gemv_perm:      y[n] = sum_j x[perm[j]] * ŵ[n,j]
 *   w4a16_gemm_perm:      Y[m,n] = sum_j X[m, perm[j]] * ŵ[n,j]  (VALU
 *                         path up to w4a16_valu_max_m() rows; above, X is
 *                         first copied in the order perm, 2 M K bytes taken
 *                         on the stream from a pool the library keeps per
 *                         device, and the matrix-core GEMM runs on the copy;
 *                         under graph capture the VALU path, which allocates
 *                         nothing; w4a16_linear takes a caller workspace)
 * A NULL perm with K > 0 is W4A16_ERR_INVALID_ARG; outputs must not overlap
 * perm. */
int w4a16_quantize_perm(const uint16_t* W, const int32_t* perm, int64_t N, int64_t K,
                        uint32_t* packed, uint16_t* scales, void* stream);
int w4a16_gemv_perm(const uint16_t* x, const int32_t* perm, const uint32_t* packed,
                    const uint16_t* scales, int64_t N, int64_t K, uint16_t* y, void* stream);
int w4a16_gemm_perm(const uint16_t* X, int64_t M, const int32_t* perm, const uint32_t* packed,
                    const uint16_t* scales, int64_t N, int64_t K, uint16_t* Y, void* stream);

/* ---- Asymmetric INT4 ([QUANT] sub-section 2, asymmetric equations: scale
 * (max - min) / 15, zero point z = -round(min / s), codes clamp(round(w / s)
 * + z, 0, 15), INT4 range [0, 15]; the same section's guidance puts skewed
 * weight distributions, e.g. the FFN down projection, on this form).
 * Per group of `group` elements along K (32, 64, 128, 256, or the whole row
 * with W4A16_PER_CHANNEL):
 *     s    = fp16 RNE of (max - min) / 15 (exact max - min)
 *     z    = -RNE(min / s), an integer, against the stored fp16 s
 *     q    = clamp(RNE(w / s) + z, 0, 15), stored as the nibble itself
 *            (no offset), element 8j+i in bits 4i..4i+3 of word j
 *     ŵ    = s * (q - z)
 *   a group whose scale rounds to 0 (range below 2^-24 * 7.5) stores s = 0,
 *   z = 0 and q = 0.  z lies in [0, 15] when the group holds both signs;
 *   a one-signed group with a narrow range can have |z| up to 32752.
 *   zeros: int16 [N, K/group], laid out like the scales (N*(K/group)*2
 *   bytes = w4a16_scales_bytes_g), 2-byte aligned.
 *   perm: NULL (columns in W's order) or the act-order column order as for
 *   the *_perm functions (device int32 [K], 16-byte aligned).
 *   w4a16_quantize_asym: W fp16 [N, K] -> packed, scales, zeros (outputs must
 *                        not overlap each other, W or perm)
 *   w4a16_gemv_asym:     y[n] = sum_j x[perm[j]] * ŵ[n,j]      (x[j] without perm)
 *   w4a16_gemm_asym:     Y[m,n] = sum_j X[m, perm[j]] * ŵ[n,j]  (the VALU
 *                        path for M <= w4a16_valu_max_m(), the matrix cores
 *                        above; with perm as for w4a16_gemm_perm)
 * Errors as for w4a16_gemm_g; a NULL zeros with K > 0 is
 * W4A16_ERR_INVALID_ARG; Y must not overlap zeros. */
int w4a16_quantize_asym(const uint16_t* W, const int32_t* perm, int64_t N, int64_t K,
                        int64_t group, uint32_t* packed, uint16_t* scales, int16_t* zeros,
                        void* stream);
int w4a16_gemv_asym(const uint16_t* x, const int32_t* perm, const uint32_t* packed,
                    const uint16_t* scales, const int16_t* zeros, int64_t N, int64_t K,
                    int64_t group, uint16_t* y, void* stream);
int w4a16_gemm_asym(const uint16_t* X, int64_t M, const int32_t* perm, const uint32_t* packed,
                    const uint16_t* scales, const int16_t* zeros, int64_t N, int64_t K,
                    int64_t group, uint16_t* Y, void* stream);

/* Asymmetric prefill with K split over blocks ([BENCH] §一/§二, 512-token
 * prompt; [QUANT] sub-section 2, asymmetric INT4): w4a16_gemm_asym without
 * perm, with a caller workspace, for the shapes that
 * w4a16_gemm_asym_workspace_bytes reports a non-zero size for (group 128,
 * more than 64 rows, K > N, too few 64 x 256 output tiles for the compute
 * units, at least three K slices).  Block (tile, z) takes one slice of K
 * and stores its fp32 partial tile in the workspace; a second kernel on the
 * same stream adds the slices in slice order (deterministic) and writes Y.
 * Other shapes run exactly as w4a16_gemm_asym and ignore the workspace.
 * Same accuracy bound as w4a16_gemm_asym; the sum order of split shapes
 * differs, so their results are not bit-identical to the unsplit kernel's.
 *   workspace  DEVICE, 256-byte aligned, at least
 *              w4a16_gemm_asym_workspace_bytes(M, N, K, group) bytes, owned by
 *              the caller, in use until the call's work on the stream has
 *              finished (stream-ordered calls and graph replays may share
 *              it; no initial contents needed); it must not overlap X, Y or
 *              the weights.
 * w4a16_gemm_asym_workspace_bytes returns 0 for shapes that do not split,
 * for invalid sizes and when the current device is not gfx950.  Errors as
 * for w4a16_gemm_asym; a workspace smaller than required is
 * W4A16_ERR_INVALID_ARG. */
size_t w4a16_gemm_asym_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t group);
int w4a16_gemm_asym_ws(const uint16_t* X, int64_t M, const uint32_t* packed,
                       const uint16_t* scales, const int16_t* zeros, int64_t N, int64_t K,
                       int64_t group, uint16_t* Y, void* workspace, size_t workspace_bytes,
                       void* stream);

/* ---- Q4_0 block layout ([QUANT] GGUF section: the type table's Q4_0
 * entry, 32 elements in 18 bytes, symmetric with one scale per block; the
 * section's Q4_0 dequantizer for the byte order; its llama.cpp part credits
 * block-major layouts with 20-30 % more memory-bound throughput on CPUs).
 * Each row of W is K/32 consecutive blocks of 18 bytes:
 *     bytes 0-1   d = fp16 RNE(absmax / 7) of the block's 32 elements,
 *                 little-endian
 *     byte 2+i    element 2i in bits 0-3, element 2i+1 in bits 4-7, each
 *                 as q + 8, q = clamp(RNE(w / d), -8, 7)
 * i.e. the symmetric quantizer at group 32, with each group's scale placed
 * in front of its 16 code bytes instead of in a separate array.
 * Ŵ[n, k] = d * q.  The blocks take N*(K/32)*18 bytes; the buffer must
 * hold w4a16_q4_0_bytes(N, K) bytes, that size rounded up to a multiple of
 * 16 (0 for bad sizes): the linear layer reads the padding with its
 * 16-byte loads and ignores it; the quantizer never writes it.
 *   w4a16_quantize_q4_0: W fp16 [N, K] (16-byte aligned) -> blocks (16-byte
 *                        aligned, not overlapping W)
 *   w4a16_gemv_q4_0:     y[n] = sum_k x[k] * Ŵ[n,k]
 *   w4a16_gemm_q4_0:     Y = X·Ŵᵀ, any M (VALU path; X rows in slices that
 *                        fit the staged-activation budget)
 * K % 128 == 0 as everywhere (else W4A16_ERR_SHAPE); the linear layer also
 * needs K <= 32768 (x is staged whole in LDS), else W4A16_ERR_INVALID_ARG.
 * X, x 16-byte aligned; Y, y 2-byte aligned and not overlapping X or the
 * blocks buffer. */
size_t w4a16_q4_0_bytes(int64_t N, int64_t K);
int w4a16_quantize_q4_0(const uint16_t* W, int64_t N, int64_t K, uint8_t* blocks, void* stream);
int w4a16_gemv_q4_0(const uint16_t* x, const uint8_t* blocks, int64_t N, int64_t K, uint16_t* y,
                    void* stream);
int w4a16_gemm_q4_0(const uint16_t* X, int64_t M, const uint8_t* blocks, int64_t N, int64_t K,
                    uint16_t* Y, void* stream);

/* ---- Dependent decode sequence ([BENCH] §二: every decode step streams
 * the layers' matrices one after another, each fed by the one before).
 * Runs stages[0..count) as if w4a16_gemv were called on each in order on
 * `stream`, in ONE launch: stage s may read the output of any earlier stage
 * as its x (e.g. stages[s].x == stages[s-1].y).  Outputs are bit-identical
 * to separate w4a16_gemv calls.  The grid synchronizes between stages
 * through `sync`, and the weights of the next stage are already streaming
 * while the grid waits.
 *   stages   HOST array of `count` stage descriptors (copied at the call)
 *   count    0 .. W4A16_CHAIN_MAX (0 enqueues nothing)
 *   sync     DEVICE buffer of W4A16_CHAIN_SYNC_WORDS uint32, owned by the
 *            caller, all zero before the first call; every call leaves it
 *            zero again.  Word W4A16_CHAIN_ERR_WORD becomes non-zero (and
 *            stays so) if a wait between stages ever gives up; it is never
 *            cleared by the library.  Calls sharing one `sync` buffer must not
 *            overlap in time (stream-ordered calls are fine).
 * Per stage: 128 <= K <= 32768, K % 128 == 0, 1 <= N <= 2^20; x, packed
 * 16-byte aligned; scales, y 2-byte aligned; y must not overlap any
 * stage's packed or scales, or its own stage's x (outputs of different
 * stages may alias each other and later stages' inputs: stages run in
 * order).
 * The GPU must be otherwise idle enough for the grid (sized from occupancy)
 * to be co-resident, as on a dedicated decode stream. */
#define W4A16_CHAIN_MAX 64
#define W4A16_CHAIN_SYNC_WORDS 1024
#define W4A16_CHAIN_ERR_WORD 0

typedef struct {
    const uint16_t* x;       /* fp16 [K] */
    const uint32_t* packed;  /* uint32 [N, K/8] */
    const uint16_t* scales;  /* fp16 [N, K/128] */
    uint16_t* y;             /* fp16 [N] */
    int64_t N;
    int64_t K;
} w4a16_gemv_stage;

int w4a16_gemv_chain(const w4a16_gemv_stage* stages, int count, uint32_t* sync, void* stream);

/* w4a16_gemv_chain for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same stages, outputs and rules, with the counters in the
 * library's own array instead of a caller buffer.
 *   status   DEVICE uint32, 4-byte aligned, owned by the caller: written by
 *            every call, 0 when every wait between stages completed, non-zero
 *            when one gave up (the grid was not co-resident; outputs may then
 *            be stale).  Must not overlap any stage's tensors.
 * The array is W4A16_CHAIN_SYNC_WORDS uint32 per GPU, zero when the library
 * is loaded and returned to zero (error word included) by every call; it
 * lives until the process ends.  The limit is the one of w4a16_gemv_chain:
 * count above W4A16_CHAIN_MAX is W4A16_ERR_INVALID_ARG.  Nothing is
 * allocated and no memory is cleared from the host (no memset node).  All
 * calls of a process on one GPU share its array: calls that overlap in time
 * on one GPU (e.g. on two streams) race and must not be made; stream-ordered
 * calls and graph replays are fine. */
int w4a16_gemv_chain_noalloc(const w4a16_gemv_stage* stages, int count, uint32_t* status,
                             void* stream);

/* ---- The linear layer with every option in one call (the forms above
 * are special cases of it): [QUANT] sub-section 3 granularity (group 32,
 * 64, 128, 256 or W4A16_PER_CHANNEL), sub-section 2 asymmetric weights
 * (zeros non-NULL: int16 [N, K/group], ŵ = s (q - z); NULL: symmetric
 * offset-binary codes, ŵ = s q), GPTQ section act order (perm non-NULL:
 * device int32 [K], Y[m,n] = sum_j X[m, perm[j]] ŵ[n,j], an index outside
 * [0, K) reads 0; NULL: Y = X Ŵᵀ).  algo: W4A16_ALGO_* (AUTO picks by M
 * as w4a16_gemm does; VALU and MFMA force a kernel family, every family
 * meets the accuracy bound of w4a16_gemm).
 * workspace: NULL, or device memory of at least
 * w4a16_linear_workspace_bytes(M, K, perm != NULL) bytes (16-byte aligned,
 * apart from every operand) that holds the act-order copy of X on the
 * matrix-core path, so that the call allocates nothing and can be captured
 * in a graph; with NULL the copy comes from the library's per-device pool
 * (and a capturing stream takes the VALU path).  The workspace is in use
 * until the call's work on the stream has finished.  Returns as
 * w4a16_gemm_g / w4a16_gemm_asym; a workspace smaller than required is
 * W4A16_ERR_INVALID_ARG.  w4a16_linear_workspace_bytes is 2 M K with a perm
 * (has_perm != 0), else 0 (0 for invalid sizes). */
size_t w4a16_linear_workspace_bytes(int64_t M, int64_t K, int has_perm);
int w4a16_linear(const uint16_t* X, int64_t M, const int32_t* perm, const uint32_t* packed,
                 const uint16_t* scales, const int16_t* zeros, int64_t N, int64_t K,
                 int64_t group, uint16_t* Y, int algo, void* workspace, size_t workspace_bytes,
                 void* stream);

/* Largest M that W4A16_ALGO_AUTO sends to the VALU path. */
int64_t w4a16_valu_max_m(void);

/* Static description of a status code (never NULL). */
const char* w4a16_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* W4A16_H */

"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Bar:
  * packed codes and scales: bit-exact;
  * outputs: |y - y_ref| <= 1e-3 * sum_k |x_k w_k| + max(2^-10 |y_ref|, 2^-24)
    per element (oracle.tolerance; the floor is one fp16 subnormal step);
  * one-hot activations: bit-exact fp16(s*q).
Inputs: seeded draws of weight_only_int4_gemv_amd.inputs (layer-like weights
with 0.1 % outliers, N(0,1) activations).  Weights given to the linear
kernels are the oracle's own packed codes and scales.
"""
import functools
import sys

import numpy as np
import pytest

import oracle
from weight_only_int4_gemv_amd import inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def say(msg):
    print("[case] " + msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def w4():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    from weight_only_int4_gemv_amd import w4a16
    w4a16.library()                       # must be built; no fallback
    return w4a16


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def dev(a: np.ndarray):
    t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to("cuda")


def packed_to_dev(p: np.ndarray):
    return dev(p.view(np.int32))


def scales_to_dev(s: np.ndarray):
    return dev(s.view(np.float16))


# ------------------------------------------------------------------ quantize

def check_quantize(w4, orc, W: np.ndarray, name: str):
    N, K = W.shape
    say("quantize %s N=%d K=%d" % (name, N, K))
    pg, sg = w4.quantize(dev(W))
    torch.cuda.synchronize()
    po, so = orc.quantize(W)
    got_p = pg.cpu().numpy().view(np.uint32)
    got_s = sg.cpu().numpy().view(np.uint16)
    bad_s = np.argwhere(got_s != so)
    assert bad_s.size == 0, "%s: %d scales differ, first at %s" % (name, len(bad_s), bad_s[0])
    bad_p = np.argwhere(got_p != po)
    assert bad_p.size == 0, "%s: %d words differ, first at %s (%#x vs %#x)" % (
        name, len(bad_p), bad_p[0], got_p[tuple(bad_p[0])], po[tuple(bad_p[0])])


@pytest.mark.parametrize("N,K,seed", [(1, 128, 1), (3, 256, 2), (37, 384, 3), (129, 1152, 4),
                                      (4096, 4096, 0)])
def test_quantize_bit_exact(w4, orc, N, K, seed):
    W = inputs.weight(N, K, seed=seed)
    check_quantize(w4, orc, W, "seed %d" % seed)


@pytest.mark.parametrize("name,K,N", inputs.LLAMA3_8B[::3] + inputs.QWEN25_7B[4:]
                         + inputs.FFN_70B)
def test_quantize_bit_exact_layer_shapes(w4, orc, name, K, N):
    W = inputs.weight(N, K, seed=inputs.matrix_seed(2, 0, K * 7 + N))
    check_quantize(w4, orc, W, name)


def test_quantize_every_fp16_absmax(w4, orc):
    """One group per positive finite fp16 value a (absmax a, sign alternating,
    the rest of the group a ramp below a): scale rounding, subnormal scales,
    clamping and ties over the whole fp16 range."""
    a_bits = np.arange(1, 0x7C00, dtype=np.uint16)
    a = a_bits.view(np.float16).astype(np.float32)
    ramp = np.linspace(-1.0, 1.0, 127, dtype=np.float32)
    W = np.empty((a_bits.size, 128), dtype=np.float16)
    W[:, 1:] = (a[:, None] * ramp[None, :]).astype(np.float16)
    W[:, 0] = np.where(np.arange(a_bits.size) % 2 == 0, 1, -1) * a.astype(np.float16)
    check_quantize(w4, orc, W, "every fp16 absmax")


def test_quantize_hand_worked_groups(w4, orc):
    import json
    import oracle_pins
    spec = json.load(open(oracle_pins.GOLDEN))
    W = np.zeros((len(spec["groups"]), 128), dtype=np.float16)
    for r, g in enumerate(spec["groups"]):
        for k, v in g["nonzero"].items():
            W[r, int(k)] = np.float16(v)
    say("quantize hand-worked groups")
    pg, sg = w4.quantize(dev(W))
    got_p = pg.cpu().numpy().view(np.uint32)
    got_s = sg.cpu().numpy().view(np.uint16)
    for r, g in enumerate(spec["groups"]):
        assert got_s[r, 0] == int(g["scale_bits"], 16), g["name"]
        for j in range(16):
            want = int(g["words"].get(str(j), g["words"]["rest"]), 16)
            assert got_p[r, j] == want, (g["name"], j, hex(got_p[r, j]), hex(want))


def test_quantize_edge_values(w4, orc):
    rng = np.random.default_rng(77)
    W = (rng.standard_normal((64, 512)) * 0.02).astype(np.float16)
    W[0] = 0                                                  # all zero
    W[1] = np.float16(-0.0)                                   # negative zeros
    W[2, :128] = np.float16(65504.0)                          # largest fp16
    W[2, 128:256] = np.float16(-65504.0)
    W[3] = (rng.standard_normal(512) * 1e-6).astype(np.float16)   # subnormal scales
    W[4, :128] = np.uint16(1).view(np.float16)               # smallest subnormal
    W[5, :128] = np.uint16(3).view(np.float16)               # scale rounds to 0
    W[5, 128:256] = np.uint16(4).view(np.float16)            # smallest non-zero scale
    check_quantize(w4, orc, W, "edge values")


def test_quantize_ties_and_near_ties(w4, orc):
    """Quotients w/s that are exact half-integers (round half to even) and
    values one fp16 step either side of them, for scales 2^e (e = -14..0)
    and for scales that are not powers of two."""
    rows = []
    rng = np.random.default_rng(78)
    for e in range(-14, 1):
        s = 2.0 ** e
        a = np.float16(7 * s)                      # absmax: s = fp16(a / 7) = 2^e
        ties = np.array([(k + 0.5) * s for k in range(-7, 6)], dtype=np.float64)
        vals = np.concatenate([ties, -ties]).astype(np.float16)
        up = np.nextafter(vals, np.float16(np.inf))
        dn = np.nextafter(vals, np.float16(-np.inf))
        g = np.concatenate([vals, up, dn])
        g = np.resize(np.concatenate([g, rng.permutation(g)]), 127)
        rows.append(np.concatenate([[a], g]).astype(np.float16))
    for a in (0.1, 0.37, 1.9, 5.3, 200.0):         # s not a power of two
        s = float(np.float16(np.float16(a) / 7.0))
        ties = np.array([(k + 0.5) * s for k in range(-7, 6)])
        vals = ties.astype(np.float16)             # ties up to fp16 rounding
        up = np.nextafter(vals, np.float16(np.inf))
        g = np.resize(np.concatenate([vals, up, -vals, -up]), 127)
        rows.append(np.concatenate([[np.float16(a)], g]).astype(np.float16))
    W = np.stack(rows)
    W = np.concatenate([W, W[:, ::-1]], axis=1)    # K = 256
    check_quantize(w4, orc, np.ascontiguousarray(W), "ties")


def test_quantize_empty_and_deterministic(w4, orc):
    say("quantize empty")
    p, s = w4.quantize(torch.empty((0, 256), dtype=torch.float16, device="cuda"))
    assert p.shape == (0, 32) and s.shape == (0, 2)
    W = inputs.weight(300, 640, seed=12)
    p1, s1 = w4.quantize(dev(W))
    p2, s2 = w4.quantize(dev(W))
    assert torch.equal(p1, p2) and torch.equal(s1, s2)


# -------------------------------------------------------------------- linear

def run_linear(w4, X16: np.ndarray, packed: np.ndarray, scales: np.ndarray, algo):
    Xd = dev(X16)
    if algo == "gemv":
        return w4.gemv(Xd[0], packed_to_dev(packed), scales_to_dev(scales)).cpu().numpy()[None]
    return w4.gemm(Xd, packed_to_dev(packed), scales_to_dev(scales), algo=algo).cpu().numpy()


@functools.lru_cache(maxsize=3)
def layer(N, K, wseed):
    """(W, packed, scales) of one seeded layer, quantized by the oracle."""
    W = inputs.weight(N, K, seed=list(wseed) if isinstance(wseed, tuple) else wseed)
    packed, scales = oracle.get().quantize(W)
    return W, packed, scales


def check_linear(w4, orc, M, N, K, seed, algo, name="", full_limit=6e8):
    """seed: (weight seed, activation seed) or one seed for both."""
    say("linear %s M=%d N=%d K=%d algo=%s" % (name, M, N, K, algo))
    wseed, xseed = seed if isinstance(seed, tuple) else (seed, [1000, seed] if isinstance(
        seed, int) else [1000] + list(seed))
    _, packed, scales = layer(N, K, tuple(wseed) if isinstance(wseed, list) else wseed)
    X = inputs.activation(M, K, seed=xseed)
    Y = run_linear(w4, X, packed, scales, algo)
    torch.cuda.synchronize()
    assert Y.shape == (M, N)
    if M * N * K <= full_limit:
        Yref, Yabs = orc.matmul(X, packed, scales)
        got = Y.astype(np.float64)
    else:
        rng = np.random.default_rng(M * 1000003 + N * 7 + K)
        cols = np.unique(np.concatenate([[0, N - 1], rng.integers(0, N, 96)]))
        rows = np.unique(np.concatenate([[0, M - 1], rng.integers(0, M, 8)]))
        rr, cc = np.meshgrid(rows, cols, indexing="ij")
        ys, ya = orc.matmul_sampled(X, packed, scales, rr.ravel(), cc.ravel())
        Yref, Yabs = ys.reshape(rr.shape), ya.reshape(rr.shape)
        got = Y[rr, cc].astype(np.float64)
    tol = oracle.tolerance(Yref, Yabs)
    err = np.abs(got - Yref)
    bad = np.argwhere(~(err <= tol))
    assert bad.size == 0, "%s: %d outputs out of tolerance, first %s: got %r want %r tol %r" % (
        name, len(bad), bad[0], got[tuple(bad[0])], Yref[tuple(bad[0])], tol[tuple(bad[0])])
    return float((err / np.maximum(tol, 1e-30)).max())


@pytest.mark.parametrize("N,K", [(1, 128), (7, 256), (37, 384), (300, 1152), (1000, 2048),
                                 (2053, 4224), (5, 512), (1003, 1536), (37, 18944),
                                 (32771, 512), (33003, 1536)])
@pytest.mark.parametrize("algo", ["gemv", "valu", "mfma"])
def test_linear_m1_small_and_ragged(w4, orc, N, K, algo):
    """Ragged N.  K = 512 and 1536 (16 and 48 chunks of 32) with at least 128
    rows per compute unit run the GEMV with four rows side by side, 16 lanes
    each (fewer rows, or K = 18944, keep 64 lanes per row)."""
    check_linear(w4, orc, 1, N, K, seed=[5, N, K], algo=algo)


def test_gemv_config1_single_layer(w4, orc):
    """4096 x 4096, M = 1, seed 0 (the single-layer case)."""
    check_linear(w4, orc, 1, 4096, 4096, seed=0, algo="gemv", name="4096x4096")


LAYER_SHAPES = [("llama " + n, K, N) for n, K, N in inputs.LLAMA3_8B] + \
               [("llama qkv", 4096, 6144), ("llama gate_up", 4096, 28672)] + \
               [("qwen " + n, K, N) for n, K, N in inputs.QWEN25_7B] + \
               [("qwen qkv", 3584, 4608), ("qwen gate_up", 3584, 37888)] + \
               [("70b gate_up", 8192, 28672)]


@pytest.mark.parametrize("name,K,N", LAYER_SHAPES, ids=[s[0] for s in LAYER_SHAPES])
def test_gemv_decode_layer_shapes(w4, orc, name, K, N):
    check_linear(w4, orc, 1, N, K, seed=[2, 0, N * 7 + K], algo="gemv", name=name)


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 8, 16, 32])
@pytest.mark.parametrize("K,N", [(4096, 14336), (14336, 4096)])
@pytest.mark.parametrize("algo", ["valu", "mfma", "auto"])
def test_batched_decode_ffn(w4, orc, M, K, N, algo):
    check_linear(w4, orc, M, N, K, seed=([4, K], [4, K, M]), algo=algo, name="ffn")


@pytest.mark.parametrize("M", [2, 3, 9, 15, 16, 17, 31, 33, 48, 64, 65, 127, 129, 200])
@pytest.mark.parametrize("algo", ["valu", "mfma"])
def test_gemm_ragged_m(w4, orc, M, algo):
    check_linear(w4, orc, M, 300, 640, seed=([6], [6, M]), algo=algo, name="ragged")


@pytest.mark.parametrize("M", [3, 16, 17, 33, 64])
@pytest.mark.parametrize("N,K", [(5, 128), (40, 256), (50, 5120), (1000, 4224)])
def test_mfma_long_rows(w4, orc, M, N, K):
    """K > N: the K groups are split over waves (fewer groups than waves at
    K = 128 and 256), ragged N and M tiles."""
    check_linear(w4, orc, M, N, K, seed=([8, N, K], [8, N, K, M]), algo="mfma", name="long rows")


@pytest.mark.parametrize("M,N,K", [(4, 1001, 8320), (3, 9002, 14464), (4, 64, 16384),
                                   (1, 64, 512), (2, 4100, 14336), (4, 4096, 14336),
                                   (4, 14336, 4096), (4, 3584, 18944), (4, 700, 19456)])
def test_mfma4_k_split(w4, orc, M, N, K):
    """The 4x4x4 matrix-core GEMV with two waves per row group (few row
    groups for the CUs, or x above 64 KiB): ragged N, an odd step count
    (the second wave's last step lies past K), several batches per block
    (N = 9002), x of 128 KiB, of 148 KiB (the Qwen-2.5-7B down projection)
    and of exactly 152 KiB (the largest staged), a single step (the second
    wave only pads), and the one-wave-per-row-group launch as a control."""
    check_linear(w4, orc, M, N, K, seed=([49, N, K], [49, N, K, M]), algo="mfma",
                 name="4x4x4 k split")


BATCHED_SHAPES = [(1, 128), (100, 2176), (4104, 2176), (9000, 1152), (30000, 640),
                  (40000, 256), (300, 14464)]


@pytest.mark.parametrize("M", [5, 12, 16, 20, 32])
@pytest.mark.parametrize("N,K", BATCHED_SHAPES)
def test_batched_rows_and_chunks(w4, orc, M, N, K):
    """Batched decode kernel: rows per block from 1 to 128 (and beyond, more
    blocks than compute units at N = 40000), every wave-grid class, partial
    16-row tiles, K ragged against the 1024/2048-wide X chunks (one group,
    a chunk plus one group, 113 groups), 16- and 32-row X tiles."""
    check_linear(w4, orc, M, N, K, seed=([9, N, K], [9, N, K, M]), algo="mfma", name="batched")


@pytest.mark.parametrize("K,N", [(4096, 14336), (14336, 4096), (8192, 28672)])
def test_prefill_512(w4, orc, K, N):
    check_linear(w4, orc, 512, N, K, seed=[5, K, N], algo="auto", name="prefill")


def whole_reference(orc, X16: np.ndarray, packed: np.ndarray, scales: np.ndarray):
    """(Y, Yabs) for every output of a workload-size product: the oracle's
    exact dequantized weights (binary64 s*q) multiplied by X in a float64
    matrix product (a library primitive), and |X| times |W| for the
    tolerance.  The product's own rounding, at most about K 2^-53 sum|x w|,
    is below 1e-9 of the allowance."""
    What = orc.dequantize(packed, scales)
    Xf = X16.astype(np.float64)
    Y = Xf @ What.T
    np.abs(What, out=What)
    Yabs = np.abs(Xf) @ What.T
    return Y, Yabs


WHOLE_CASES = [(32, 4096, 14336, "auto"), (32, 14336, 4096, "auto"),
               (16, 14336, 4096, "auto"), (512, 4096, 14336, "auto"),
               (512, 14336, 4096, "auto"), (512, 8192, 28672, "auto")]


@pytest.mark.parametrize("M,K,N,algo", WHOLE_CASES,
                         ids=["M%d-%dx%d" % (c[0], c[1], c[2]) for c in WHOLE_CASES])
def test_workload_size_whole_output(w4, orc, M, K, N, algo):
    """Batched decode (M = 16, 32 on the FFN shapes) and the 512-token
    prefill (both FFN shapes and the 70B FFN) compared on EVERY output, in
    the launch configuration the benchmark times (the automatic choice), so
    that each block-tile family and every tile of these grids is checked."""
    say("whole output M=%d K=%d N=%d algo=%s" % (M, K, N, algo))
    _, packed, scales = layer(N, K, (7, K, N))
    X = inputs.activation(M, K, seed=[7, K, N, M])
    Y = run_linear(w4, X, packed, scales, algo)
    torch.cuda.synchronize()
    assert Y.shape == (M, N)
    Yref, Yabs = whole_reference(orc, X, packed, scales)
    tol = oracle.tolerance(Yref, Yabs)
    err = np.abs(Y.astype(np.float64) - Yref)
    bad = np.argwhere(~(err <= tol))
    assert bad.size == 0, "%d of %d outputs out of tolerance, first %s: got %r want %r tol %r" % (
        len(bad), Y.size, bad[0], Y[tuple(bad[0])], Yref[tuple(bad[0])], tol[tuple(bad[0])])


@pytest.mark.parametrize("M,N,K", [(520, 6600, 384), (129, 33000, 256), (512, 32776, 128),
                                   (250, 14400, 256), (100, 14400, 384), (70, 3000, 384),
                                   (300, 4100, 1152)])
def test_prefill_wide_tiles_ragged(w4, orc, M, N, K):
    """Every prefill block tile on 256 compute units: 128 x 256 blocks (the
    first three shapes), 128 x 128 and 64 x 128 blocks with two waves over
    K, and 64 x 64 blocks; M and N ragged against them, few groups, and
    canary words around Y that must survive (no store outside Y)."""
    _, packed, scales = layer(N, K, (31, M, N, K))
    X = inputs.activation(M, K, seed=[32, M, N, K])
    pad = 4096
    buf = torch.full((pad + M * N + pad,), float("nan"), dtype=torch.float16, device="cuda")
    Y = buf[pad:pad + M * N].view(M, N)
    say("wide tiles M=%d N=%d K=%d" % (M, N, K))
    w4.gemm(dev(X), packed_to_dev(packed), scales_to_dev(scales), algo="mfma", Y=Y)
    torch.cuda.synchronize()
    b = buf.cpu().numpy().view(np.uint16)
    nan_bits = np.float16("nan").view(np.uint16)
    assert (b[:pad] == nan_bits).all() and (b[pad + M * N:] == nan_bits).all()
    Yref, Yabs = orc.matmul(X, packed, scales)
    err = np.abs(Y.cpu().numpy().astype(np.float64) - Yref)
    bad = np.argwhere(~(err <= oracle.tolerance(Yref, Yabs)))
    assert bad.size == 0, "%d outputs out of tolerance, first %s" % (len(bad), bad[0])


@pytest.mark.parametrize("M,N,K,algo", [(1, 64, 512, "gemv"), (3, 64, 512, "valu"),
                                         (3, 64, 512, "mfma"), (16, 64, 512, "mfma"),
                                         (40, 64, 512, "mfma"), (65, 64, 512, "mfma"),
                                         (512, 64, 512, "mfma"), (256, 16384, 256, "mfma"),
                                         (65, 64, 1024, "mfma"), (512, 8192, 1024, "mfma")])
def test_largest_fp16_weights_stay_finite(w4, orc, M, N, K, algo):
    """Groups whose absmax is the largest finite fp16 (65504) get s = 9360,
    and s * 7 = 65520 is a tie that rounds to infinity in fp16.  Every kernel
    family (GEMV, VALU, 4x4x4, batched, streaming, both tiled block shapes)
    must keep these weights finite and match the oracle within tolerance
    (the kernels that form fp16 weights clamp them to +-65504: error 16 in
    65520, 2.4e-4 relative).  K = 1024 gives rows of eight scales, which the
    tiled kernel's scale scan reads 16 bytes at a time."""
    W = inputs.weight(N, K, seed=[35, N, K])
    W[::3, 5] = np.float16(65504.0)
    W[1::3, K // 2 + 3] = np.float16(-65504.0)
    W[2::7, K - 7] = np.float16(65472.0)                  # s = 9352: 7 s = 65464 stays finite
    packed, scales = orc.quantize(W)
    assert (scales.view(np.uint16) == 0x7092).any()      # s = 9360 present
    X = (inputs.activation(M, K, seed=[36, M]).astype(np.float32) * 2.0 ** -8).astype(np.float16)
    say("largest weights %s M=%d N=%d K=%d" % (algo, M, N, K))
    Y = run_linear(w4, X, packed, scales, algo)
    torch.cuda.synchronize()
    Yref, Yabs = orc.matmul(X, packed, scales)
    assert np.isfinite(Yref).all() and np.abs(Yref).max() < 60000
    got = Y.astype(np.float64)
    assert np.isfinite(got).all(), "%d non-finite outputs" % (~np.isfinite(got)).sum()
    bad = np.argwhere(~(np.abs(got - Yref) <= oracle.tolerance(Yref, Yabs)))
    assert bad.size == 0, "%d outputs out of tolerance, first %s" % (len(bad), bad[0])


def test_tiled_rows_past_32bit_offsets_fall_back(w4, orc):
    """Rows longer than 2^22 elements do not fit the tiled kernel's 32-bit
    block offsets; with 65 rows of X (past the batched and streaming
    kernels) such a product runs on the VALU path and still matches."""
    M, N, K = 65, 8, (1 << 22) + 128
    check_linear(w4, orc, M, N, K, seed=([33, K], [34, K]), algo="mfma", name="long K")


def test_70b_ffn_decode(w4, orc):
    check_linear(w4, orc, 1, 28672, 8192, seed=[5, 1, 8192], algo="auto", name="70b m1")


# -------------------------------------------------------------- exact cases

@pytest.mark.parametrize("algo", ["gemv", "valu", "mfma", "mfma-4rows"])
def test_one_hot_activations_are_exact(w4, orc, algo):
    """x = e_k reproduces fp16(s*q) of column k exactly, for every k of two
    groups: checks nibble order, word order and scale indexing."""
    N, K = 96, 256
    W = inputs.weight(N, K, seed=21)
    packed, scales = orc.quantize(W)
    What = orc.dequantize(packed, scales)
    want = What.astype(np.float16)                     # RNE of the exact s*q
    for k0 in range(0, K, 64):
        ks = list(range(k0, k0 + 64))
        say("one-hot %s k=%d..%d" % (algo, ks[0], ks[-1]))
        if algo == "gemv":
            rows = []
            for k in ks:
                x = np.zeros((1, K), dtype=np.float16)
                x[0, k] = 1
                rows.append(run_linear(w4, x, packed, scales, "gemv")[0])
            Y = np.stack(rows)
        elif algo == "mfma-4rows":
            # four rows per call: the 4x4x4 matrix-core GEMV
            parts = []
            for i in range(0, len(ks), 4):
                X = np.zeros((4, K), dtype=np.float16)
                X[np.arange(4), ks[i:i + 4]] = 1
                parts.append(run_linear(w4, X, packed, scales, "mfma"))
            Y = np.concatenate(parts)
        else:
            X = np.zeros((len(ks), K), dtype=np.float16)
            X[np.arange(len(ks)), ks] = 1
            Y = run_linear(w4, X, packed, scales, algo)
        np.testing.assert_array_equal(Y.view(np.uint16), want[:, ks].T.view(np.uint16))


@pytest.mark.parametrize("algo", ["gemv", "valu", "mfma"])
def test_scaled_identity(w4, orc, algo):
    """W = c I with c = 7 * 2^-6: s = 2^-6, q = 7 on the diagonal, so
    y = c x within tolerance."""
    K = 512
    W = np.zeros((K, K), dtype=np.float16)
    W[np.arange(K), np.arange(K)] = np.float16(0.109375)
    packed, scales = orc.quantize(W)
    X = inputs.activation(3 if algo != "gemv" else 1, K, seed=22)
    say("scaled identity %s" % algo)
    Y = run_linear(w4, X, packed, scales, algo).astype(np.float64)
    want = 0.109375 * X.astype(np.float64)
    tol = 1e-3 * np.abs(want) + 2.0 ** -10 * np.abs(want)
    assert (np.abs(Y - want) <= tol).all()


@pytest.mark.parametrize("algo", ["gemv", "valu", "mfma"])
def test_k_zero_gives_zeros(w4, algo):
    say("K=0 %s" % algo)
    packed = torch.empty((5, 0), dtype=torch.int32, device="cuda")
    scales = torch.empty((5, 0), dtype=torch.float16, device="cuda")
    if algo == "gemv":
        y = w4.gemv(torch.empty((0,), dtype=torch.float16, device="cuda"), packed, scales)
    else:
        y = w4.gemm(torch.empty((2, 0), dtype=torch.float16, device="cuda"), packed, scales,
                    algo=algo)
    assert torch.count_nonzero(y).item() == 0


def test_empty_m_and_n(w4):
    say("empty M / N")
    packed = torch.zeros((4, 16), dtype=torch.int32, device="cuda")
    scales = torch.zeros((4, 1), dtype=torch.float16, device="cuda")
    Y = w4.gemm(torch.empty((0, 128), dtype=torch.float16, device="cuda"), packed, scales)
    assert Y.shape == (0, 4)
    Y = w4.gemm(torch.zeros((3, 128), dtype=torch.float16, device="cuda"),
                torch.zeros((0, 16), dtype=torch.int32, device="cuda"),
                torch.zeros((0, 1), dtype=torch.float16, device="cuda"))
    assert Y.shape == (3, 0)


@pytest.mark.parametrize("M,algo", [(1, "gemv"), (3, "valu"), (3, "mfma"), (20, "mfma"),
                                    (64, "mfma"), (130, "mfma")])
def test_outputs_stay_inside_their_buffer(w4, orc, M, algo):
    """Canary words around Y must survive (no out-of-bounds stores)."""
    N, K = 333, 768
    W, X = inputs.weight_and_activation(N, K, M, seed=[23, M])
    packed, scales = orc.quantize(W)
    pad = 4096
    buf = torch.full((pad + M * N + pad,), float("nan"), dtype=torch.float16, device="cuda")
    Y = buf[pad:pad + M * N].view(M, N)
    say("canary %s M=%d" % (algo, M))
    if algo == "gemv":
        w4.gemv(dev(X)[0], packed_to_dev(packed), scales_to_dev(scales), y=Y[0])
    else:
        w4.gemm(dev(X), packed_to_dev(packed), scales_to_dev(scales), algo=algo, Y=Y)
    b = buf.cpu().numpy().view(np.uint16)
    nan_bits = np.float16("nan").view(np.uint16)
    assert (b[:pad] == nan_bits).all() and (b[pad + M * N:] == nan_bits).all()
    assert not np.isnan(buf[pad:pad + M * N].cpu().numpy()).any()


@pytest.mark.parametrize("M,algo,N", [(1, "gemv", 2048), (8, "valu", 2048), (4, "mfma", 2048),
                                      (32, "mfma", 2048), (16, "mfma", 1024), (512, "mfma", 2048)])
def test_deterministic_and_stream_ordered(w4, orc, M, algo, N):
    K = 2048
    W, X = inputs.weight_and_activation(N, K, M, seed=[24, M])
    packed, scales = orc.quantize(W)
    pd, sd, Xd = packed_to_dev(packed), scales_to_dev(scales), dev(X)
    say("determinism %s M=%d" % (algo, M))
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    outs = []
    for s in (torch.cuda.current_stream(), side, side):
        with torch.cuda.stream(s):
            if algo == "gemv":
                outs.append(w4.gemv(Xd[0], pd, sd)[None])
            else:
                outs.append(w4.gemm(Xd, pd, sd, algo=algo))
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[1], outs[2])


# ------------------------------------------------------- group size as a parameter

GROUP_SIZES = [32, 64, 256]


@pytest.mark.parametrize("group", GROUP_SIZES)
@pytest.mark.parametrize("N,K", [(37, 768), (129, 1536), (4096, 4096), (300, 14336)])
def test_quantize_group_sizes_bit_exact(w4, orc, group, N, K):
    """w4a16_quantize_g against the oracle at the same group size: every code
    and scale bit-exact, including an all-zero and a tiny-scale group."""
    say("quantize group=%d N=%d K=%d" % (group, N, K))
    W = inputs.weight(N, K, seed=[21, group, N, K])
    W[0, :group] = np.float16(0)
    W[min(1, N - 1), group:2 * group] *= np.float16(1e-4)
    pg, sg = w4.quantize(dev(W), group=group)
    torch.cuda.synchronize()
    po, so = orc.quantize(W, group=group)
    got_s = sg.cpu().numpy().view(np.uint16)
    got_p = pg.cpu().numpy().view(np.uint32)
    assert got_s.shape == (N, K // group)
    bad_s = np.argwhere(got_s != so)
    assert bad_s.size == 0, "%d scales differ, first at %s" % (len(bad_s), bad_s[0])
    bad_p = np.argwhere(got_p != po)
    assert bad_p.size == 0, "%d words differ, first at %s" % (len(bad_p), bad_p[0])


def check_linear_group(w4, orc, M, N, K, group, seed, algo=None):
    say("linear group=%d M=%d N=%d K=%d algo=%s" % (group, M, N, K, algo))
    W = inputs.weight(N, K, seed=[22, group, N, K])
    packed, scales = orc.quantize(W, group=group)
    X = inputs.activation(M, K, seed=seed)
    if M == 1 and algo == "gemv":
        Y = w4.gemv(dev(X)[0], packed_to_dev(packed), scales_to_dev(scales)).cpu().numpy()[None]
    else:
        Y = w4.gemm(dev(X), packed_to_dev(packed), scales_to_dev(scales), algo=algo).cpu().numpy()
    torch.cuda.synchronize()
    assert Y.shape == (M, N)
    Yref, Yabs = orc.matmul(X, packed, scales, group=group)
    tol = oracle.tolerance(Yref, Yabs)
    err = np.abs(Y.astype(np.float64) - Yref)
    bad = np.argwhere(~(err <= tol))
    assert bad.size == 0, "%d outputs out of tolerance, first %s: got %r want %r" % (
        len(bad), bad[0], Y[tuple(bad[0])], Yref[tuple(bad[0])])


@pytest.mark.parametrize("group", GROUP_SIZES)
@pytest.mark.parametrize("M,algo", [(1, "gemv"), (2, None), (3, "valu"), (8, "valu"),
                                    (13, "valu"), (8, None)])
@pytest.mark.parametrize("N,K", [(300, 1536), (1001, 4096), (64, 14336)])
def test_linear_group_sizes(w4, orc, group, M, algo, N, K):
    """GEMV and the VALU GEMM (both launch families: whole-x staging for the
    persistent kernel, K slices for M = 8) at other group sizes, and the
    automatic choice above two rows (the tiled matrix-core kernel)."""
    check_linear_group(w4, orc, M, N, K, group, seed=[23, group, M, N, K], algo=algo)


@pytest.mark.parametrize("group", GROUP_SIZES)
def test_linear_group_sizes_layer_shape(w4, orc, group):
    """M = 1 on the LLaMA-3-8B gate shape (4096 x 14336) at each group size."""
    check_linear_group(w4, orc, 1, 14336, 4096, group, seed=[24, group], algo="gemv")


@pytest.mark.parametrize("group", GROUP_SIZES)
def test_group_sizes_one_hot_exact(w4, orc, group):
    """One-hot activations select fp16(s[k // group] * q[k]) bit-exactly: the
    scale of every group is read for the right codes."""
    N, K = 24, 1024
    W = inputs.weight(N, K, seed=[25, group])
    packed, scales = orc.quantize(W, group=group)
    ks = np.arange(0, K, 7)
    X = np.zeros((len(ks), K), dtype=np.float16)
    X[np.arange(len(ks)), ks] = np.float16(1.0)
    say("one-hot group=%d" % group)
    for m0 in range(0, len(ks), 8):
        Y = w4.gemm(dev(X[m0:m0 + 8]), packed_to_dev(packed), scales_to_dev(scales)).cpu().numpy()
        torch.cuda.synchronize()
        deq = orc.dequantize(packed, scales, group=group)[:, ks[m0:m0 + 8]].T
        want = deq.astype(np.float16)
        assert (Y.view(np.uint16) == want.view(np.uint16)).all()


# ------------------------------------------------------- act-order column order

def perm_of(kind: str, K: int, seed) -> np.ndarray:
    rng = np.random.default_rng(seed)
    if kind == "identity":
        return np.arange(K, dtype=np.int32)
    if kind == "reverse":
        return np.arange(K - 1, -1, -1, dtype=np.int32)
    return rng.permutation(K).astype(np.int32)


@pytest.mark.parametrize("kind", ["identity", "reverse", "random"])
@pytest.mark.parametrize("N,K", [(37, 384), (300, 4096), (129, 14336)])
def test_quantize_act_order_bit_exact(w4, orc, kind, N, K):
    """w4a16_quantize_perm = the oracle's quantizer on W[:, perm], bit for bit."""
    say("quantize act-order %s N=%d K=%d" % (kind, N, K))
    W = inputs.weight(N, K, seed=[31, N, K])
    perm = perm_of(kind, K, [31, K])
    pg, sg = w4.quantize(dev(W), perm=dev(perm))
    torch.cuda.synchronize()
    po, so = orc.quantize(np.ascontiguousarray(W[:, perm]))
    assert (sg.cpu().numpy().view(np.uint16) == so).all()
    assert (pg.cpu().numpy().view(np.uint32) == po).all()


@pytest.mark.parametrize("kind", ["identity", "random"])
@pytest.mark.parametrize("M,algo", [(1, None), (2, None), (3, "valu"), (8, "valu"), (13, "valu"),
                                    (8, None)])
@pytest.mark.parametrize("N,K", [(300, 1536), (1001, 4096), (64, 14336)])
def test_linear_act_order(w4, orc, kind, M, algo, N, K):
    """y = X[:, perm] . Ŵpᵀ on the VALU path (persistent kernel with whole-x
    staging, and K slices for M = 8, 13 at K = 14336) and the automatic
    choice above two rows (gathered copy of X, matrix cores), against the
    oracle on the gathered activations."""
    say("linear act-order %s M=%d N=%d K=%d algo=%s" % (kind, M, N, K, algo))
    W = inputs.weight(N, K, seed=[32, N, K])
    perm = perm_of(kind, K, [32, K])
    packed, scales = orc.quantize(np.ascontiguousarray(W[:, perm]))
    X = inputs.activation(M, K, seed=[32, M, N, K])
    if M == 1:
        Y = w4.gemv(dev(X)[0], packed_to_dev(packed), scales_to_dev(scales),
                    perm=dev(perm)).cpu().numpy()[None]
    else:
        Y = w4.gemm(dev(X), packed_to_dev(packed), scales_to_dev(scales),
                    perm=dev(perm), algo=algo).cpu().numpy()
    torch.cuda.synchronize()
    Yref, Yabs = orc.matmul(np.ascontiguousarray(X[:, perm]), packed, scales)
    tol = oracle.tolerance(Yref, Yabs)
    err = np.abs(Y.astype(np.float64) - Yref)
    bad = np.argwhere(~(err <= tol))
    assert bad.size == 0, "%d outputs out of tolerance, first %s" % (len(bad), bad[0])


def test_act_order_one_hot_exact(w4, orc):
    """A one-hot x at position k selects stored column inv[k]: fp16(s*q) exactly."""
    N, K = 40, 512
    W = inputs.weight(N, K, seed=[33])
    perm = perm_of("random", K, [33])
    packed, scales = orc.quantize(np.ascontiguousarray(W[:, perm]))
    deq = orc.dequantize(packed, scales)
    inv = np.argsort(perm)
    say("act-order one-hot")
    for k in [0, 1, 127, 128, 300, 511]:
        x = np.zeros(K, dtype=np.float16)
        x[k] = np.float16(1.0)
        y = w4.gemv(dev(x), packed_to_dev(packed), scales_to_dev(scales), perm=dev(perm))
        torch.cuda.synchronize()
        want = deq[:, inv[k]].astype(np.float16)
        assert (y.cpu().numpy().view(np.uint16) == want.view(np.uint16)).all(), k


def test_act_order_out_of_range_index_reads_zero(w4, orc):
    """perm entries outside [0, K) read as 0 (documented), in both the
    quantizer and the GEMV; no access leaves the buffers."""
    N, K = 16, 256
    W = inputs.weight(N, K, seed=[34])
    X = inputs.activation(1, K, seed=[34, 1])
    perm = perm_of("random", K, [34]).copy()
    perm[5], perm[130], perm[200] = -1, K, 1 << 30
    Wz = np.ascontiguousarray(W[:, np.clip(perm, 0, K - 1)])
    Wz[:, [5, 130, 200]] = np.float16(0)
    pg, sg = w4.quantize(dev(W), perm=dev(perm))
    torch.cuda.synchronize()
    po, so = orc.quantize(Wz)
    assert (pg.cpu().numpy().view(np.uint32) == po).all()
    assert (sg.cpu().numpy().view(np.uint16) == so).all()
    Xz = np.ascontiguousarray(X[:, np.clip(perm, 0, K - 1)])
    Xz[:, [5, 130, 200]] = np.float16(0)
    y = w4.gemv(dev(X)[0], pg, sg, perm=dev(perm)).cpu().numpy()[None]
    torch.cuda.synchronize()
    Yref, Yabs = orc.matmul(Xz, po, so)
    assert (np.abs(y.astype(np.float64) - Yref) <= oracle.tolerance(Yref, Yabs)).all()


# ------------------------------------------------------------ asymmetric INT4

def asym_weight(N, K, seed, plant=True, extremes=False):
    """Skewed layer-like weights; with plant, the first rows get groups that
    exercise every branch of the asymmetric path: one-signed groups whose
    zero point lies beyond +-1000 (about -2700 and +1550), a one-signed group
    near z = -300, a constant group (range 0), an all-zero group, a range that
    rounds the fp16 scale to 0, exact ties, and with extremes the fp16
    extremes (quantizer tests only: outputs of such a row overflow fp16)."""
    W = inputs.weight_skewed(N, K, seed=seed)
    if not plant:
        return W
    r = np.arange(K, dtype=np.float64)
    if N > 0:
        W[0] = (20.0 + (r % 8) / 64.0).astype(np.float16)                   # z ~ -2700
    if N > 1:
        W[1] = (-12.0 - (r % 16) / 128.0).astype(np.float16)                # z = 1551
    if N > 2:
        W[2] = (10.0 + (r % 128) / 254.0).astype(np.float16)                # z ~ -300
    if N > 3:
        W[3, :] = np.float16(0.75)                                           # constant
        W[3, 64:] = np.float16(0)                                            # all zero
    if N > 4:
        W[4, :] = np.float16(2.0 ** -24)
        W[4, ::64] = np.float16(0)                                           # s16 = 0
    if N > 5 and extremes:
        W[5, :] = np.float16(0)
        W[5, 0], W[5, 1] = np.float16(65504.0), np.float16(-65504.0)         # widest range
    if N > 6:
        # range 7.5 -> s = 0.5, z = 3: 2.25 and 2.75 are exact ties of w / s
        W[6, :] = np.float16(2.25)
        W[6, 0::32], W[6, 1::32], W[6, 2::32] = np.float16(-1.5), np.float16(6.0), np.float16(2.75)
    return W


def check_quantize_asym(w4, orc, W, group, perm=None, name=""):
    N, K = W.shape
    say("quantize asym %s group=%d N=%d K=%d perm=%s" % (name, group, N, K, perm is not None))
    pg, sg, zg = w4.quantize_asym(dev(W), group=group,
                                  perm=None if perm is None else dev(perm))
    torch.cuda.synchronize()
    Wo = W if perm is None else np.ascontiguousarray(W[:, perm])
    po, so, zo = orc.quantize_asym(Wo, group=group)
    got_s = sg.cpu().numpy().view(np.uint16)
    got_z = zg.cpu().numpy()
    got_p = pg.cpu().numpy().view(np.uint32)
    bad = np.argwhere(got_s != so)
    assert bad.size == 0, "%d scales differ, first at %s" % (len(bad), bad[0])
    bad = np.argwhere(got_z != zo)
    assert bad.size == 0, "%d zeros differ, first at %s: %d vs %d" % (
        len(bad), bad[0], got_z[tuple(bad[0])], zo[tuple(bad[0])])
    bad = np.argwhere(got_p != po)
    assert bad.size == 0, "%d words differ, first at %s (%#x vs %#x)" % (
        len(bad), bad[0], got_p[tuple(bad[0])], po[tuple(bad[0])])
    return po, so, zo


@pytest.mark.parametrize("group", [32, 64, 128, 256])
@pytest.mark.parametrize("N,K", [(7, 256), (37, 768), (129, 1536), (4096, 4096), (300, 14336)])
def test_quantize_asym_bit_exact(w4, orc, group, N, K):
    """w4a16_quantize_asym against the oracle: codes, scales and zero points
    bit-exact, planted edge groups included."""
    check_quantize_asym(w4, orc, asym_weight(N, K, [41, group, N, K], extremes=True), group)


def test_quantize_asym_every_range(w4, orc):
    """One group per positive finite fp16 value v with min 0 and max v (and
    one with min -v and max 0): the scale RNE(v / 15) at every binade,
    subnormal and zero scales included, and z at both ends."""
    v = np.arange(1, 0x7C00, dtype=np.uint16).view(np.float16)
    G = len(v)
    W = np.zeros((2 * G, 128), dtype=np.float16)
    W[:G, 5] = v
    W[G:, 9] = -v
    W[:G, 17] = (v.astype(np.float64) * 0.37).astype(np.float16)
    W[G:, 17] = (-v.astype(np.float64) * 0.61).astype(np.float16)
    check_quantize_asym(w4, orc, W, 128, name="every range")


def test_quantize_asym_ties_and_zero_parity(w4, orc):
    """Groups whose elements sit exactly on half-integers of w / s: the code
    is rint(w / s) + z, which differs from rint(w / s + z) when z is odd
    (rint(-2.5) + 3 = 1, rint(0.5) = 0), for every z in [0, 15] and scales
    1, 1/8 and 3; and groups whose min / s is itself a tie (z from a rounded
    tie).  Elements a quarter off the half-integers check the ordinary
    rounding beside them."""
    rows, want = [], []
    for s in (1.0, 0.125, 3.0):
        for z in range(0, 16):
            base = -z * s                      # min, so that z = -rint(min / s)
            vals = [base, base + 15 * s]       # range 15 s: the scale is s
            for off in (0.5, 0.25, 0.75):
                vals += [(j + off - z) * s for j in range(15)]
            vals += [base] * (128 - len(vals))
            rows.append(vals)
            want.append((s, z))
        for m in range(0, 8):                  # min / s = -(m + 1/2): a tie for z
            base = -(m + 0.5) * s
            vals = [base, base + 15 * s] + [(j + 0.5) * s + base for j in range(15)]
            vals += [base] * (128 - len(vals))
            rows.append(vals)
            want.append((s, m + (m & 1)))      # rint(m + 1/2), half to even
    W = np.array(rows, dtype=np.float64)
    assert np.array_equal(W.astype(np.float16).astype(np.float64), W)   # exact in fp16
    _, so, zo = orc.quantize_asym(W.astype(np.float16), group=128)
    assert np.array_equal(so.view(np.float16)[:, 0].astype(np.float64), [s for s, _ in want])
    assert np.array_equal(zo[:, 0], [z for _, z in want])
    check_quantize_asym(w4, orc, W.astype(np.float16), 128, name="ties")


@pytest.mark.parametrize("kind", ["reverse", "random"])
@pytest.mark.parametrize("group", [64, 128])
def test_quantize_asym_act_order(w4, orc, kind, group):
    W = asym_weight(129, 4096, [42, group], extremes=True)
    check_quantize_asym(w4, orc, W, group, perm=perm_of(kind, 4096, [42, group]), name=kind)


def check_linear_asym(w4, orc, M, N, K, group, seed, perm_kind=None, plant=True, algo=None):
    say("linear asym group=%d M=%d N=%d K=%d perm=%s algo=%s" % (group, M, N, K, perm_kind,
                                                                  algo))
    W = asym_weight(N, K, seed, plant=plant)
    perm = None if perm_kind is None else perm_of(perm_kind, K, seed)
    Wo = W if perm is None else np.ascontiguousarray(W[:, perm])
    packed, scales, zeros = orc.quantize_asym(Wo, group=group)
    X = inputs.activation(M, K, seed=[1000] + list(seed))
    pd, sd, zd = packed_to_dev(packed), scales_to_dev(scales), dev(zeros)
    permd = None if perm is None else dev(perm)
    if M == 1:
        Y = w4.gemv_asym(dev(X)[0], pd, sd, zd, perm=permd).cpu().numpy()[None]
    else:
        Y = w4.gemm_asym(dev(X), pd, sd, zd, perm=permd, algo=algo).cpu().numpy()
    torch.cuda.synchronize()
    assert Y.shape == (M, N)
    Xo = X if perm is None else np.ascontiguousarray(X[:, perm])
    Yref, Yabs = orc.matmul_asym(Xo, packed, scales, zeros, group=group)
    tol = oracle.tolerance(Yref, Yabs)
    err = np.abs(Y.astype(np.float64) - Yref)
    bad = np.argwhere(~(err <= tol))
    assert bad.size == 0, "%d outputs out of tolerance, first %s: got %r want %r tol %r" % (
        len(bad), bad[0], Y[tuple(bad[0])], Yref[tuple(bad[0])], tol[tuple(bad[0])])


@pytest.mark.parametrize("group", [32, 128, 256])
@pytest.mark.parametrize("M,algo", [(1, None), (2, None), (3, "valu"), (8, "valu"),
                                    (13, "valu"), (3, None), (13, None)])
@pytest.mark.parametrize("N,K", [(300, 1536), (1001, 4096), (64, 14336)])
def test_linear_asym(w4, orc, group, M, algo, N, K):
    """Asymmetric GEMV / VALU GEMM for every M family (persistent kernel with
    whole-x staging; K slices for M = 8, 13 at K = 14336) and the automatic
    choice above two rows (matrix cores), planted groups with |z| > 1000
    (the chunk-sum correction) included."""
    check_linear_asym(w4, orc, M, N, K, group, [43, group, M, N, K], algo=algo)


@pytest.mark.parametrize("M", [3, 16, 17, 32, 33, 64, 65, 200, 512])
@pytest.mark.parametrize("N,K", [(300, 4096), (64, 14336), (1000, 1152)])
def test_linear_asym_matrix_cores(w4, orc, M, N, K):
    """M > 2 at group 128 runs on the matrix cores: the batched decode kernel
    up to 32 rows, the tiled kernel above (64-row and 128-row prefill
    tiles), planted |z| > 1000 groups (the ones-MFMA correction) included."""
    check_linear_asym(w4, orc, M, N, K, 128, [47, M, N, K])


@pytest.mark.parametrize("M", [5, 16, 20, 32])
@pytest.mark.parametrize("N,K", [(4104, 2176), (9000, 1152), (30000, 1152), (300, 14464)])
def test_linear_asym_batched_wave_grids(w4, orc, M, N, K):
    """Asymmetric weights on the batched decode kernel: every wave-grid class
    (rows per block 17, 36 and 118: two, four and eight 16-row tiles), K
    ragged against the staged X chunks, 16- and 32-row X tiles, planted
    |z| > 1000 groups."""
    check_linear_asym(w4, orc, M, N, K, 128, [48, M, N, K])


@pytest.mark.parametrize("M,N,K", [(512, 8192, 1024), (300, 11000, 640), (250, 7200, 384),
                                   (200, 3000, 512), (512, 4096, 3072)])
def test_linear_asym_prefill_fp16_weights(w4, orc, M, N, K):
    """Prefill-sized asymmetric products whose blocks all take the fp16
    weight copy (skewed layer-like weights: scales below 64, zero points in
    [0, 15]) on each prefill block tile (128 x 128 blocks when they fill the
    compute units, 64 x 128 blocks of 32-column wave tiles and 64 x 64 blocks
    with two waves over K), M and N ragged."""
    check_linear_asym(w4, orc, M, N, K, 128, [51, M, N, K], plant=False)


@pytest.mark.parametrize("M,N,K", [(520, 11620, 512), (512, 8000, 512), (300, 6000, 1152)],
                         ids=["128x256", "128x128", "64x128"])
def test_linear_asym_wide_prefill_common_and_slow_launches(w4, orc, M, N, K):
    """Prefill shapes with planted groups (|z| > 1000, scale 0, ties) in
    several column blocks, on each asymmetric prefill tiling: where 128 x
    256 blocks fill the compute units the common-copy launch leaves the
    blocks with such groups to the slow-copy launch, which decides over the
    same 256 columns; with fewer blocks (128 x 128 and 64 x 128 block tiles)
    each block picks its copy.  Every output is computed exactly once and
    meets the bound."""
    W = asym_weight(N, K, [52, N, K])
    W[[N // 40 * 1 + 300, N // 2 + 1, N - 9]] = W[[0, 1, 2]]   # planted rows in more column blocks
    packed, scales, zeros = orc.quantize_asym(W, group=128)
    X = inputs.activation(M, K, seed=[52, M])
    say("asym wide prefill M=%d N=%d K=%d" % (M, N, K))
    Y = w4.gemm_asym(dev(X), packed_to_dev(packed), scales_to_dev(scales), dev(zeros))
    torch.cuda.synchronize()
    Yref, Yabs = orc.matmul_asym(X, packed, scales, zeros, group=128)
    got = Y.cpu().numpy().astype(np.float64)
    bad = np.argwhere(~(np.abs(got - Yref) <= oracle.tolerance(Yref, Yabs)))
    assert bad.size == 0, "%d outputs out of tolerance, first %s" % (len(bad), bad[0])


@pytest.mark.parametrize("M,N,K", [(65, 300, 1024), (65, 300, 512), (512, 8192, 1024),
                                   (520, 11620, 512), (512, 4096, 1024), (450, 3584, 2048)])
def test_linear_asym_large_scales(w4, orc, M, N, K):
    """Asymmetric weights with scales of 64 and more (the tiled kernel's
    slow copy: fp16 weights s * (n - zc) clamped to +-65504), including
    groups that hold +-65504, against the oracle (rows of eight scales:
    the 16-byte scale scan; of four: the 2-byte one; every block shape:
    64 x 64, 128 x 128, the two-launch 128 x 256, 64 x 128 with 32-column
    wave tiles)."""
    rng = np.random.default_rng([49, M, N, K])
    W = (rng.standard_normal((N, K)) * 3000.0).astype(np.float16)
    W[::5, 7] = np.float16(65504.0)
    W[1::5, K - 9] = np.float16(-65504.0)
    packed, scales, zeros = orc.quantize_asym(W, group=128)
    assert (scales.view(np.float16).astype(np.float32) >= 64.0).any()
    X = (inputs.activation(M, K, seed=[50, M]).astype(np.float32) * 2.0 ** -12).astype(np.float16)
    say("asym large scales M=%d N=%d K=%d" % (M, N, K))
    Y = w4.gemm_asym(dev(X), packed_to_dev(packed), scales_to_dev(scales), dev(zeros))
    torch.cuda.synchronize()
    Yref, Yabs = orc.matmul_asym(X, packed, scales, zeros, group=128)
    assert np.abs(Yref).max() < 30000
    got = Y.cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    bad = np.argwhere(~(np.abs(got - Yref) <= oracle.tolerance(Yref, Yabs)))
    assert bad.size == 0, "%d outputs out of tolerance, first %s" % (len(bad), bad[0])


@pytest.mark.parametrize("name,K,N", [("llama down", 14336, 4096), ("llama gate", 4096, 14336),
                                      ("qwen down", 18944, 3584)])
def test_linear_asym_layer_shapes(w4, orc, name, K, N):
    """M = 1 on full decode layer shapes, group 128 (the down projection is
    the skewed layer asymmetric INT4 is meant for)."""
    check_linear_asym(w4, orc, 1, N, K, 128, [44, N, K], plant=False)


@pytest.mark.parametrize("M,algo", [(1, None), (4, "valu"), (4, None), (130, None)])
def test_linear_asym_act_order(w4, orc, M, algo):
    check_linear_asym(w4, orc, M, 515, 4096, 128, [45, M], perm_kind="random", algo=algo)


def test_asym_one_hot_exact(w4, orc):
    """One-hot activations select fp16(s * (q - z)) bit-exactly where
    |q - z| < 2^13 (the fp32 product s * (q - z) is then exact)."""
    N, K = 24, 1024
    W = asym_weight(N, K, [46], plant=False)
    packed, scales, zeros = orc.quantize_asym(W, group=64)
    ks = np.arange(0, K, 5)
    X = np.zeros((len(ks), K), dtype=np.float16)
    X[np.arange(len(ks)), ks] = np.float16(1.0)
    assert np.abs(zeros.astype(np.int64)).max() < 2 ** 12
    say("asym one-hot")
    pd, sd, zd = packed_to_dev(packed), scales_to_dev(scales), dev(zeros)
    deq = orc.dequantize_asym(packed, scales, zeros, group=64)
    for m0 in range(0, len(ks), 8):
        Y = w4.gemm_asym(dev(X[m0:m0 + 8]), pd, sd, zd).cpu().numpy()
        torch.cuda.synchronize()
        want = deq[:, ks[m0:m0 + 8]].T.astype(np.float16)
        assert (Y.view(np.uint16) == want.view(np.uint16)).all()


def test_asym_empty_and_k_zero(w4):
    say("asym empty / K = 0")
    p, s, z = w4.quantize_asym(torch.empty((0, 256), dtype=torch.float16, device="cuda"))
    assert p.shape == (0, 32) and s.shape == (0, 2) and z.shape == (0, 2)
    Y = w4.gemm_asym(torch.empty((3, 0), dtype=torch.float16, device="cuda"),
                     torch.empty((5, 0), dtype=torch.int32, device="cuda"),
                     torch.empty((5, 0), dtype=torch.float16, device="cuda"),
                     torch.empty((5, 0), dtype=torch.int16, device="cuda"))
    torch.cuda.synchronize()
    assert Y.shape == (3, 5) and (Y.cpu().numpy() == 0).all()


# ------------------------------------------------------------ Q4_0 blocks

Q40_QUANT_SHAPES = [(1, 128), (37, 384), (129, 1152), (4096, 4096), (300, 14336)]


@pytest.mark.parametrize("N,K", Q40_QUANT_SHAPES)
def test_quantize_q4_0_bit_exact(w4, orc, N, K):
    """w4a16_quantize_q4_0 against the oracle byte for byte (all-zero and
    tiny-scale blocks planted), and against the GPU's own group-32 split
    layout: each block is that layout's scale followed by its 16 code bytes."""
    say("quantize q4_0 N=%d K=%d" % (N, K))
    W = inputs.weight(N, K, seed=[51, N, K])
    W[0, :32] = np.float16(0)
    W[N - 1, K - 32:] *= np.float16(1e-4)
    bg = w4.quantize_q4_0(dev(W))
    pg, sg = w4.quantize(dev(W), group=32)
    torch.cuda.synchronize()
    got = bg.cpu().numpy()
    want = orc.quantize_q4_0(W)
    bad = np.argwhere(got != want)
    assert bad.size == 0, "%d bytes differ, first at %s" % (len(bad), bad[0])
    split = np.concatenate([sg.cpu().numpy().view(np.uint8).reshape(N, K // 32, 2),
                            pg.cpu().numpy().view(np.uint8).reshape(N, K // 32, 16)], axis=2)
    assert (split.reshape(N, -1) == got).all()


def q4_0_to_dev(w4, blocks: np.ndarray):
    """Oracle blocks into a device buffer with the library's 16-byte padding."""
    N = blocks.shape[0]
    out = w4.q4_0_blocks(N, blocks.shape[1] // 18 * 32)
    out.copy_(torch.from_numpy(np.ascontiguousarray(blocks)))
    return out


def check_linear_q4_0(w4, orc, M, N, K, seed):
    say("linear q4_0 M=%d N=%d K=%d" % (M, N, K))
    W = inputs.weight(N, K, seed=[52] + list(seed))
    blocks = orc.quantize_q4_0(W)
    X = inputs.activation(M, K, seed=[53] + list(seed))
    bd = q4_0_to_dev(w4, blocks)
    if M == 1:
        Y = w4.gemv_q4_0(dev(X)[0], bd).cpu().numpy()[None]
    else:
        Y = w4.gemm_q4_0(dev(X), bd).cpu().numpy()
    torch.cuda.synchronize()
    assert Y.shape == (M, N)
    Yref, Yabs = orc.matmul_q4_0(X, blocks)
    tol = oracle.tolerance(Yref, Yabs)
    err = np.abs(Y.astype(np.float64) - Yref)
    bad = np.argwhere(~(err <= tol))
    assert bad.size == 0, "%d outputs out of tolerance, first %s: got %r want %r tol %r" % (
        len(bad), bad[0], Y[tuple(bad[0])], Yref[tuple(bad[0])], tol[tuple(bad[0])])


@pytest.mark.parametrize("M", [1, 2, 3, 5, 8, 13])
@pytest.mark.parametrize("N,K", [(1, 128), (7, 256), (37, 384), (300, 1152), (1001, 4096),
                                 (515, 3584), (64, 14336), (33, 32768)])
def test_linear_q4_0(w4, orc, M, N, K):
    """Rows of 18-byte blocks start at every 2-byte offset mod 16 (K = 384:
    216-byte rows), partial last wave steps (K = 384, 1152, 3584), odd N
    (a row group with one row), K up to the 32768 limit, M in slices."""
    check_linear_q4_0(w4, orc, M, N, K, [M, N, K])


@pytest.mark.parametrize("name,K,N", [("llama gate", 4096, 14336), ("llama down", 14336, 4096),
                                      ("qwen gate", 3584, 18944), ("qwen down", 18944, 3584)])
def test_gemv_q4_0_layer_shapes(w4, orc, name, K, N):
    check_linear_q4_0(w4, orc, 1, N, K, [7, N, K])


def test_q4_0_one_hot_exact(w4, orc):
    """One-hot x selects fp16(d * q) bit-exactly: block scale and nibble order."""
    N, K = 40, 1024
    W = inputs.weight(N, K, seed=[54])
    blocks = orc.quantize_q4_0(W)
    deq = orc.dequantize_q4_0(blocks, K)
    ks = np.arange(0, K, 3)
    X = np.zeros((len(ks), K), dtype=np.float16)
    X[np.arange(len(ks)), ks] = np.float16(1.0)
    say("q4_0 one-hot")
    bd = q4_0_to_dev(w4, blocks)
    for m0 in range(0, len(ks), 8):
        Y = w4.gemm_q4_0(dev(X[m0:m0 + 8]), bd).cpu().numpy()
        torch.cuda.synchronize()
        want = deq[:, ks[m0:m0 + 8]].T.astype(np.float16)
        assert (Y.view(np.uint16) == want.view(np.uint16)).all()


def test_q4_0_outputs_stay_inside_their_buffer(w4, orc):
    N, K, M = 333, 1152, 3
    W, X = inputs.weight_and_activation(N, K, M, seed=[55])
    blocks = orc.quantize_q4_0(W)
    pad = 4096
    buf = torch.full((pad + M * N + pad,), float("nan"), dtype=torch.float16, device="cuda")
    Y = buf[pad:pad + M * N].view(M, N)
    say("q4_0 canary")
    w4.gemm_q4_0(dev(X), q4_0_to_dev(w4, blocks), Y=Y)
    b = buf.cpu().numpy().view(np.uint16)
    nan_bits = np.float16("nan").view(np.uint16)
    assert (b[:pad] == nan_bits).all() and (b[pad + M * N:] == nan_bits).all()
    assert not np.isnan(buf[pad:pad + M * N].cpu().numpy()).any()


def test_q4_0_empty_and_k_zero(w4):
    say("q4_0 empty / K = 0")
    b = w4.quantize_q4_0(torch.empty((0, 256), dtype=torch.float16, device="cuda"))
    assert b.shape == (0, 144)
    Y = w4.gemm_q4_0(torch.empty((3, 0), dtype=torch.float16, device="cuda"),
                     torch.empty((5, 0), dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    assert Y.shape == (3, 5) and (Y.cpu().numpy() == 0).all()
    with pytest.raises(ValueError):                  # storage without the padding
        w4.gemv_q4_0(torch.zeros(128, dtype=torch.float16, device="cuda"),
                     torch.zeros((1, 72), dtype=torch.uint8, device="cuda"))


# ------------------------------------------------------ split-K batched decode

WS_CASES = [(5, 14336, 4096), (8, 14336, 4096), (16, 14336, 4096), (17, 14336, 4096),
            (32, 14336, 4096), (16, 18944, 3584), (32, 18944, 3584), (9, 16384, 4000),
            (32, 2048, 300), (3, 14336, 4096), (16, 4096, 14336)]


@pytest.mark.parametrize("M,K,N", WS_CASES, ids=["M%d-%dx%d" % c for c in WS_CASES])
def test_gemm_ws_split_k(w4, orc, M, K, N):
    """w4a16_gemm_ws on the long-K batched-decode shapes that it splits over
    blocks (and shapes it does not split, which run as w4a16_gemm): every
    output within the tolerance of the oracle, the workspace counters back
    to zero after the call, and a second call bit-identical to the first
    (the slices are summed in a fixed order)."""
    say("gemm_ws M=%d K=%d N=%d" % (M, K, N))
    _, packed, scales = layer(N, K, (8, K, N))
    X = inputs.activation(M, K, seed=[8, K, N, M])
    nws = w4.library().w4a16_gemm_workspace_bytes(M, N, K)
    ws = w4.gemm_workspace(M, N, K)
    Xd, pd, sd = dev(X), packed_to_dev(packed), scales_to_dev(scales)
    Y1 = w4.gemm_ws(Xd, pd, sd, ws).cpu().numpy()
    Y2 = w4.gemm_ws(Xd, pd, sd, ws).cpu().numpy()
    torch.cuda.synchronize()
    assert np.array_equal(Y1.view(np.uint16), Y2.view(np.uint16)), "not deterministic"
    if nws:
        assert int(ws[:4096].view(torch.int32).abs().sum().item()) == 0, "counters not zero"
    if M * N * K <= 6e8:
        Yref, Yabs = orc.matmul(X, packed, scales)
    else:
        Yref, Yabs = whole_reference(orc, X, packed, scales)
    tol = oracle.tolerance(Yref, Yabs)
    err = np.abs(Y1.astype(np.float64) - Yref)
    bad = np.argwhere(~(err <= tol))
    assert bad.size == 0, "%d outputs out of tolerance, first %s" % (len(bad), bad[0])


def test_gemm_ws_one_workspace_many_shapes(w4, orc):
    """One workspace, sized for the largest split, reused across split and
    unsplit shapes in any order (the counters live at a fixed place for
    every shape) and under graph replay: every result equal to the first
    call's of its shape."""
    shapes = [(16, 14336, 4096), (32, 18944, 3584), (8, 16384, 4000), (16, 4096, 14336),
              (32, 14336, 4096)]
    need = max(w4.library().w4a16_gemm_workspace_bytes(M, N, K) for M, K, N in shapes)
    assert need > 0
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    runs = []
    for M, K, N in shapes:
        _, packed, scales = layer(N, K, (8, K, N))
        X = dev(inputs.activation(M, K, seed=[9, K, N, M]))
        runs.append((X, packed_to_dev(packed), scales_to_dev(scales)))
    say("gemm_ws shared workspace")
    first = [w4.gemm_ws(X, p, s, ws).clone() for X, p, s in runs]
    for order in ([4, 3, 2, 1, 0], [1, 1, 0, 2, 4, 3]):
        for i in order:
            X, p, s = runs[i]
            got = w4.gemm_ws(X, p, s, ws)
            assert torch.equal(got.view(torch.int16), first[i].view(torch.int16)), i
    outs = [torch.empty_like(f) for f in first]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for (X, p, s), o in zip(runs, outs):
            w4.gemm_ws(X, p, s, ws, Y=o)
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        junk = torch.randn(1 << 18, device="cuda").sum()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, f) in enumerate(zip(outs, first)):
            assert torch.equal(o.view(torch.int16), f.view(torch.int16)), (rep, i)
        del junk
    assert int(ws[:4096].view(torch.int32).abs().sum().item()) == 0


def test_gemm_ws_rejects_small_workspace(w4):
    M, K, N = 16, 14336, 4096
    need = w4.library().w4a16_gemm_workspace_bytes(M, N, K)
    assert need > 4096
    X = torch.zeros((M, K), dtype=torch.float16, device="cuda")
    p = torch.zeros((N, K // 8), dtype=torch.int32, device="cuda")
    s = torch.zeros((N, K // 128), dtype=torch.float16, device="cuda")
    small = torch.zeros(need - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(w4.W4A16Error):
        w4.gemm_ws(X, p, s, small)

"""Per-channel scales (group = the whole row, W4A16_PER_CHANNEL) on the GPU
against the oracle at group = K: quantizer bit-exact (symmetric and
asymmetric, with and without the act-order column order), linear layer
within the tolerance for every M family, one-hot activations exact."""
import numpy as np
import pytest

import oracle
from weight_only_int4_gemv_amd import inputs

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def w4():
    assert torch.cuda.is_available()
    from weight_only_int4_gemv_amd import w4a16
    w4a16.library()
    return w4a16


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def say(msg):
    print("[case] " + msg, flush=True)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def planted(N, K, seed):
    W = inputs.weight(N, K, seed=seed)
    W[0] = np.float16(0)                                  # s = 0: every code 0
    if N > 1:
        W[1] *= np.float16(1e-4)                          # tiny scale (subnormal range)
    if N > 2:
        W[2, K // 3] = np.float16(-9.5)                   # a negative outlier sets the scale
    return W


@pytest.mark.parametrize("N,K", [(3, 128), (7, 256), (37, 768), (129, 1536), (1000, 4096),
                                 (300, 14336), (64, 18944), (9, 20480), (5, 32768), (5, 33024)])
def test_quantize_per_channel_bit_exact(w4, orc, N, K):
    """One pass per row (the row held in registers: up to 1024, 2048 or 4096
    chunks of 8 a row) and, past 32768 columns, the row reduction followed by
    the codes: scales and packed words bit-exact with the oracle at G = K."""
    say("quantize per channel N=%d K=%d" % (N, K))
    W = planted(N, K, [61, N, K])
    pg, sg = w4.quantize(dev(W), group=w4.PER_CHANNEL)
    torch.cuda.synchronize()
    po, so = orc.quantize(W, group=K)
    assert tuple(sg.shape) == (N, 1)
    got_s = sg.cpu().numpy().view(np.uint16)
    got_p = pg.cpu().numpy().view(np.uint32)
    bad = np.argwhere(got_s != so)
    assert bad.size == 0, "%d scales differ, first at %s" % (len(bad), bad[0])
    bad = np.argwhere(got_p != po)
    assert bad.size == 0, "%d words differ, first at %s" % (len(bad), bad[0])


@pytest.mark.parametrize("perm_kind", [None, "reverse", "random"])
@pytest.mark.parametrize("N,K", [(37, 768), (300, 4096), (20, 14336), (9, 33024)])
def test_quantize_per_channel_asym_bit_exact(w4, orc, perm_kind, N, K):
    say("quantize asym per channel N=%d K=%d perm=%s" % (N, K, perm_kind))
    W = inputs.weight_skewed(N, K, seed=[62, N, K])
    W[0] = np.float16(0.75)                               # constant row: s = 0, z = 0
    perm = None
    if perm_kind == "reverse":
        perm = np.arange(K - 1, -1, -1, dtype=np.int32)
    elif perm_kind == "random":
        perm = np.random.default_rng([62, K]).permutation(K).astype(np.int32)
    pg, sg, zg = w4.quantize_asym(dev(W), group=w4.PER_CHANNEL,
                                  perm=None if perm is None else dev(perm))
    torch.cuda.synchronize()
    Wo = W if perm is None else np.ascontiguousarray(W[:, perm])
    po, so, zo = orc.quantize_asym(Wo, group=K)
    assert np.array_equal(sg.cpu().numpy().view(np.uint16), so)
    assert np.array_equal(zg.cpu().numpy(), zo)
    assert np.array_equal(pg.cpu().numpy().view(np.uint32), po)


def check_linear(w4, orc, M, N, K, seed, algo=None, asym=False):
    say("linear per channel M=%d N=%d K=%d algo=%s asym=%s" % (M, N, K, algo, asym))
    if asym:
        W = inputs.weight_skewed(N, K, seed=seed)
        packed, scales, zeros = orc.quantize_asym(W, group=K)
    else:
        W = inputs.weight(N, K, seed=seed)
        packed, scales = orc.quantize(W, group=K)
    X = inputs.activation(M, K, seed=[1000] + list(seed))
    pd, sd = dev(packed.view(np.int32)), dev(scales.view(np.float16))
    if asym:
        zd = dev(zeros)
        Y = (w4.gemv_asym(dev(X)[0], pd, sd, zd).cpu().numpy()[None] if M == 1
             else w4.gemm_asym(dev(X), pd, sd, zd).cpu().numpy())
        Yref, Yabs = orc.matmul_asym(X, packed, scales, zeros, group=K)
    else:
        Y = (w4.gemv(dev(X)[0], pd, sd).cpu().numpy()[None] if M == 1 and algo == "gemv"
             else w4.gemm(dev(X), pd, sd, algo=algo).cpu().numpy())
        Yref, Yabs = orc.matmul(X, packed, scales, group=K)
    torch.cuda.synchronize()
    assert Y.shape == (M, N)
    tol = oracle.tolerance(Yref, Yabs)
    err = np.abs(Y.astype(np.float64) - Yref)
    bad = np.argwhere(~(err <= tol))
    assert bad.size == 0, "%d outputs out of tolerance, first %s: got %r want %r" % (
        len(bad), bad[0], Y[tuple(bad[0])], Yref[tuple(bad[0])])


@pytest.mark.parametrize("M,algo", [(1, "gemv"), (2, None), (3, None), (8, None), (13, None),
                                    (16, None), (33, None), (130, None), (8, "valu"),
                                    (13, "valu")])
@pytest.mark.parametrize("N,K", [(300, 1536), (1001, 4096), (64, 14336)])
def test_linear_per_channel(w4, orc, M, algo, N, K):
    check_linear(w4, orc, M, N, K, [63, M, N, K], algo=algo)


@pytest.mark.parametrize("K,N", [(4096, 14336), (14336, 4096), (18944, 3584)])
def test_gemv_per_channel_layer_shapes(w4, orc, K, N):
    check_linear(w4, orc, 1, N, K, [64, K, N], algo="gemv")


@pytest.mark.parametrize("M", [1, 3, 16, 40])
def test_linear_per_channel_asym(w4, orc, M):
    check_linear(w4, orc, M, 300, 4096, [65, M], asym=True)


def test_per_channel_one_hot_exact(w4, orc):
    """One-hot activations select fp16(s[n] * q[n, k]) exactly."""
    N, K = 24, 1152
    W = inputs.weight(N, K, seed=[66])
    packed, scales = orc.quantize(W, group=K)
    ks = np.arange(0, K, 11)
    X = np.zeros((len(ks), K), dtype=np.float16)
    X[np.arange(len(ks)), ks] = np.float16(1.0)
    deq = orc.dequantize(packed, scales, group=K)
    say("one-hot per channel")
    for m0 in range(0, len(ks), 8):
        Y = w4.gemm(dev(X[m0:m0 + 8]), dev(packed.view(np.int32)),
                    dev(scales.view(np.float16))).cpu().numpy()
        torch.cuda.synchronize()
        want = deq[:, ks[m0:m0 + 8]].T.astype(np.float16)
        assert (Y.view(np.uint16) == want.view(np.uint16)).all()

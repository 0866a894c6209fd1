"""Matrix-core path for every granularity ([QUANT] sub-section 3: groups of
32, 64, 256 and one scale per row), asymmetric weights at every group
([QUANT] sub-section 2), and act order ([QUANT] GPTQ section: activations
gathered in the stored column order before the GEMM), against the oracle.

Bar as in test_gpu_parity: |y - y_ref| <= oracle.tolerance per element;
one-hot activations bit-exact.  The asymmetric cases plant groups that send
a block down the exact slow copy of the tiled kernel's loop (zero points
beyond +-1000, scales of 64 and more), whose groups below 128 take the
transposed MFMA mapping.
"""
import numpy as np
import pytest

import oracle
from weight_only_int4_gemv_amd import inputs

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

PC = -1                      # one scale per row (W4A16_PER_CHANNEL)
GROUPS = [32, 64, 256, PC]


@pytest.fixture(scope="module")
def w4():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
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


def og(group, K):
    """The oracle's group argument: the whole row for per-channel scales."""
    return K if group == PC else group


def sk(group):
    """The group as a seed component (non-negative)."""
    return group if group > 0 else 1 << 20


def gname(group):
    return "per-channel" if group == PC else "g%d" % group


def check(Y, Yref, Yabs, rows=None):
    if rows is not None:
        Y = Y[rows]
    tol = oracle.tolerance(Yref, Yabs)
    err = np.abs(Y.astype(np.float64) - Yref)
    bad = np.argwhere(~(err <= tol))
    assert bad.size == 0, "%d outputs out of tolerance, first %s: got %r want %r" % (
        len(bad), bad[0], Y[tuple(bad[0])], Yref[tuple(bad[0])])


def planted_asym(N, K, seed):
    """Skewed weights; rows 0-1 one-signed and narrow (zero points about
    -2700 and +1550), row 2 with two +-480 outliers per 64 columns (scales
    of 64), the rest plain."""
    W = inputs.weight_skewed(N, K, seed=seed)
    r = np.arange(K, dtype=np.float64)
    W[0] = (20.0 + (r % 8) / 64.0).astype(np.float16)
    if N > 1:
        W[1] = (-12.0 - (r % 16) / 128.0).astype(np.float16)
    if N > 2:
        W[2] = (W[2].astype(np.float32) * 0.1).astype(np.float16)
        W[2, 0::64], W[2, 1::64] = np.float16(480.0), np.float16(-480.0)
    return W


# ---------------------------------------------------------------- symmetric

@pytest.mark.parametrize("group", GROUPS)
@pytest.mark.parametrize("M", [3, 16, 33, 64, 130])
@pytest.mark.parametrize("N,K", [(300, 1536), (1001, 4096), (64, 14336), (9000, 1024)])
def test_mfma_group_sizes(w4, orc, group, M, N, K):
    """Tiled kernel at every tile family (16, 32, 64 rows with eight waves
    over K for few columns, two across and four over K for N >= 32 per
    compute unit; 128-row prefill blocks) with the group's scale per
    32-element chunk."""
    say("mfma %s M=%d N=%d K=%d" % (gname(group), M, N, K))
    W = inputs.weight(N, K, seed=[81, sk(group), N, K])
    packed, scales = orc.quantize(W, group=og(group, K))
    X = inputs.activation(M, K, seed=[81, sk(group), M, N, K])
    Y = w4.gemm(dev(X), dev(packed.view(np.int32)), dev(scales.view(np.float16)),
                algo="mfma").cpu().numpy()
    torch.cuda.synchronize()
    check(Y, *orc.matmul(X, packed, scales, group=og(group, K)))


@pytest.mark.parametrize("group", GROUPS)
@pytest.mark.parametrize("K,N", [(4096, 14336), (14336, 4096)])
def test_mfma_group_prefill_512_sampled_rows(w4, orc, group, K, N):
    """M = 512 prefill on the LLaMA-3-8B FFN shapes (the automatic choice),
    24 rows of the output checked against the oracle."""
    say("prefill %s M=512 K=%d N=%d" % (gname(group), K, N))
    W = inputs.weight(N, K, seed=[82, sk(group), K, N])
    packed, scales = orc.quantize(W, group=og(group, K))
    X = inputs.activation(512, K, seed=[82, sk(group), K])
    Y = w4.gemm(dev(X), dev(packed.view(np.int32)), dev(scales.view(np.float16))).cpu().numpy()
    torch.cuda.synchronize()
    rows = np.random.default_rng([82, K]).choice(512, 24, replace=False)
    rows[:2] = (0, 511)
    check(Y, *orc.matmul(np.ascontiguousarray(X[rows]), packed, scales, group=og(group, K)),
          rows=rows)


@pytest.mark.parametrize("group", GROUPS)
def test_mfma_group_one_hot_exact(w4, orc, group):
    """One-hot rows through the tiled kernel (M = 40: 64-row tiles) select
    fp16(s q) of the right group bit for bit."""
    N, K = 48, 1536
    W = inputs.weight(N, K, seed=[83, sk(group)])
    packed, scales = orc.quantize(W, group=og(group, K))
    ks = np.arange(3, K, 37)[:40]
    X = np.zeros((len(ks), K), dtype=np.float16)
    X[np.arange(len(ks)), ks] = np.float16(1.0)
    say("one-hot mfma %s" % gname(group))
    Y = w4.gemm(dev(X), dev(packed.view(np.int32)), dev(scales.view(np.float16)),
                algo="mfma").cpu().numpy()
    torch.cuda.synchronize()
    want = orc.dequantize(packed, scales, group=og(group, K))[:, ks].T.astype(np.float16)
    assert (Y.view(np.uint16) == want.view(np.uint16)).all()


# --------------------------------------------------------------- asymmetric

@pytest.mark.parametrize("group", [32, 64, 128, 256, PC])
@pytest.mark.parametrize("M", [3, 16, 40, 130])
@pytest.mark.parametrize("N,K", [(200, 2048), (8300, 1024)])
def test_mfma_asym_groups_planted(w4, orc, group, M, N, K):
    """Asymmetric weights on the matrix cores at every group, with planted
    rows that send their blocks down the exact slow loop (few and many
    column tiles)."""
    say("mfma asym %s M=%d" % (gname(group), M))
    W = planted_asym(N, K, [84, sk(group)])
    packed, scales, zeros = orc.quantize_asym(W, group=og(group, K))
    X = inputs.activation(M, K, seed=[84, sk(group), M])
    Y = w4.gemm_asym(dev(X), dev(packed.view(np.int32)), dev(scales.view(np.float16)),
                     dev(zeros), algo="mfma").cpu().numpy()
    torch.cuda.synchronize()
    check(Y, *orc.matmul_asym(X, packed, scales, zeros, group=og(group, K)))


@pytest.mark.parametrize("group", [32, 64, 256, PC])
@pytest.mark.parametrize("M", [16, 512])
def test_mfma_asym_groups_plain(w4, orc, group, M):
    """Skewed weights without planted rows (the fast loop) at the FFN down
    shape; at M = 512 24 sampled rows."""
    K, N = 14336, 4096
    say("mfma asym plain %s M=%d" % (gname(group), M))
    W = inputs.weight_skewed(N, K, seed=[85, sk(group)])
    packed, scales, zeros = orc.quantize_asym(W, group=og(group, K))
    X = inputs.activation(M, K, seed=[85, sk(group), M])
    Y = w4.gemm_asym(dev(X), dev(packed.view(np.int32)), dev(scales.view(np.float16)),
                     dev(zeros)).cpu().numpy()
    torch.cuda.synchronize()
    rows = np.arange(M) if M <= 16 else np.random.default_rng([85, M]).choice(M, 24,
                                                                               replace=False)
    check(Y, *orc.matmul_asym(np.ascontiguousarray(X[rows]), packed, scales, zeros,
                              group=og(group, K)), rows=rows)


# ---------------------------------------------------------------- act order

def perm_with_holes(K, seed, holes=True):
    perm = np.random.default_rng(seed).permutation(K).astype(np.int32)
    if holes:
        perm[5], perm[K // 2 + 3], perm[K - 1] = -1, K, np.int32(2 ** 31 - 1)
    return perm


def gathered(X, perm):
    K = X.shape[1]
    ok = (perm >= 0) & (perm < K)
    Xg = np.zeros_like(X)
    Xg[:, ok] = X[:, perm[ok]]
    return Xg


@pytest.mark.parametrize("group", [128, 32, PC])
@pytest.mark.parametrize("M", [3, 16, 64, 130])
@pytest.mark.parametrize("N,K", [(300, 1536), (129, 14336)])
def test_mfma_act_order(w4, orc, group, M, N, K):
    """X gathered in the order perm (indices outside [0, K) read 0), then the
    matrix-core GEMM: the automatic choice, every tile family."""
    say("act-order mfma %s M=%d N=%d K=%d" % (gname(group), M, N, K))
    W = inputs.weight(N, K, seed=[86, sk(group), N, K])
    perm = perm_with_holes(K, [86, K])
    Wp = gathered(W, perm)
    packed, scales = orc.quantize(Wp, group=og(group, K))
    X = inputs.activation(M, K, seed=[86, M, K])
    Y = w4.gemm(dev(X), dev(packed.view(np.int32)), dev(scales.view(np.float16)),
                perm=dev(perm)).cpu().numpy()
    torch.cuda.synchronize()
    check(Y, *orc.matmul(gathered(X, perm), packed, scales, group=og(group, K)))


@pytest.mark.parametrize("group", [128, 32])
@pytest.mark.parametrize("M", [16, 130])
def test_mfma_act_order_asym(w4, orc, group, M):
    N, K = 200, 4096
    say("act-order asym mfma %s M=%d" % (gname(group), M))
    W = planted_asym(N, K, [87, sk(group)])
    perm = perm_with_holes(K, [87, K], holes=False)
    packed, scales, zeros = orc.quantize_asym(np.ascontiguousarray(W[:, perm]), group=group)
    X = inputs.activation(M, K, seed=[87, M])
    Y = w4.gemm_asym(dev(X), dev(packed.view(np.int32)), dev(scales.view(np.float16)),
                     dev(zeros), perm=dev(perm)).cpu().numpy()
    torch.cuda.synchronize()
    check(Y, *orc.matmul_asym(gathered(X, perm), packed, scales, zeros, group=group))


def test_mfma_act_order_prefill_512(w4, orc):
    """Act-order prefill at M = 512 on 4096 x 14336 (24 sampled rows)."""
    K, N, M = 4096, 14336, 512
    say("act-order prefill M=512")
    W = inputs.weight(N, K, seed=[88])
    perm = perm_with_holes(K, [88], holes=False)
    packed, scales = orc.quantize(np.ascontiguousarray(W[:, perm]))
    X = inputs.activation(M, K, seed=[88, 1])
    Y = w4.gemm(dev(X), dev(packed.view(np.int32)), dev(scales.view(np.float16)),
                perm=dev(perm)).cpu().numpy()
    torch.cuda.synchronize()
    rows = np.random.default_rng(88).choice(M, 24, replace=False)
    check(Y, *orc.matmul(gathered(X[rows], perm), packed, scales), rows=rows)


@pytest.mark.parametrize("M", [3, 130])
def test_linear_workspace_matches_pool(w4, orc, M):
    """The act-order copy in a caller workspace gives the same bits as the
    copy from the library's pool; a workspace one byte short is refused."""
    N, K = 300, 2048
    W = inputs.weight(N, K, seed=[89])
    perm = perm_with_holes(K, [89])
    packed, scales = orc.quantize(gathered(W, perm))
    X = inputs.activation(M, K, seed=[89, M])
    pd, sd, Xd, permd = (dev(packed.view(np.int32)), dev(scales.view(np.float16)), dev(X),
                         dev(perm))
    say("linear workspace M=%d" % M)
    a = w4.linear(Xd, pd, sd, perm=permd, algo="mfma")
    ws = w4.linear_workspace(M, K)
    b = w4.linear(Xd, pd, sd, perm=permd, algo="mfma", workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    check(b.cpu().numpy(), *orc.matmul(gathered(X, perm), packed, scales))
    with pytest.raises(RuntimeError):
        w4.linear(Xd, pd, sd, perm=permd, algo="mfma", workspace=ws[:-1])


def test_act_order_graph_replays(w4, orc):
    """Captured in a graph: with a workspace the gather and the matrix-core
    GEMM replay bit for bit as eager; without one the captured call takes
    the VALU path (no allocation) and still meets the tolerance."""
    N, K, M = 1536, 2304, 96
    W = inputs.weight(N, K, seed=[90])
    perm = perm_with_holes(K, [90], holes=False)
    packed, scales = orc.quantize(np.ascontiguousarray(W[:, perm]))
    X = inputs.activation(M, K, seed=[90, 1])
    pd, sd, Xd, permd = (dev(packed.view(np.int32)), dev(scales.view(np.float16)), dev(X),
                         dev(perm))
    Yref, Yabs = orc.matmul(gathered(X, perm), packed, scales)
    say("act-order graph M=%d" % M)
    ws = w4.linear_workspace(M, K)
    eager = w4.linear(Xd, pd, sd, perm=permd, workspace=ws)
    torch.cuda.synchronize()
    out = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
    out2 = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        w4.linear(Xd, pd, sd, perm=permd, workspace=ws, Y=out)
        w4.gemm(Xd, pd, sd, perm=permd, Y=out2)
    for i in range(3):
        out.fill_(float("nan"))
        out2.fill_(float("nan"))
        junk = torch.randn(1 << 20, device="cuda").sum()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), "replay %d differs from eager" % i
        check(out2.cpu().numpy(), Yref, Yabs)
        del junk

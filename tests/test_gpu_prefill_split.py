"""Prefill with K split over blocks through a caller workspace
(w4a16_gemm_ws with more than 64 rows and too few 128 x 256 output tiles for
the compute units: K > N, or K <= N with slices of at least 10 groups that
still fill the compute units), against the oracle.  Bar as in
test_gpu_parity: |y - y_ref| <= oracle.tolerance per element.
"""
import numpy as np
import pytest

import oracle
from weight_only_int4_gemv_amd import inputs

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


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


def splits(w4, M, N, K):
    return w4.library().w4a16_gemm_workspace_bytes(M, N, K) > 0


def check(Y, Yref, Yabs, rows=None):
    if rows is not None:
        Y = Y[rows]
    tol = oracle.tolerance(Yref, Yabs)
    err = np.abs(Y.astype(np.float64) - Yref)
    bad = np.argwhere(~(err <= tol))
    assert bad.size == 0, "%d outputs out of tolerance, first %s: got %r want %r" % (
        len(bad), bad[0], Y[tuple(bad[0])], Yref[tuple(bad[0])])


@pytest.mark.parametrize("M,N,K", [(65, 300, 2048), (130, 1000, 4096), (200, 3000, 14336),
                                   (300, 257, 2304)])
def test_prefill_split_parity(w4, orc, M, N, K):
    """Ragged M and N (outputs past M or N in the tiles' last rows and
    columns), 2 to 10 K slices of 8 groups and more, summed by the second
    kernel."""
    say("prefill split M=%d N=%d K=%d" % (M, N, K))
    assert splits(w4, M, N, K)
    W = inputs.weight(N, K, seed=[91, N, K])
    packed, scales = orc.quantize(W)
    X = inputs.activation(M, K, seed=[91, M, K])
    ws = w4.gemm_workspace(M, N, K, device="cuda")
    Y = w4.gemm_ws(dev(X), dev(packed.view(np.int32)), dev(scales.view(np.float16)),
                   ws).cpu().numpy()
    torch.cuda.synchronize()
    check(Y, *orc.matmul(X, packed, scales))


@pytest.mark.parametrize("M,K,N", [(512, 14336, 4096), (256, 14336, 4096), (128, 18944, 3584)])
def test_prefill_split_layer_shapes_sampled(w4, orc, M, K, N):
    """The FFN down projections of LLaMA-3-8B and Qwen-2.5-7B, 4 / 7 / 15 K
    slices (24 sampled rows, the first and last included)."""
    say("prefill split layer M=%d K=%d N=%d" % (M, K, N))
    assert splits(w4, M, N, K)
    W = inputs.weight(N, K, seed=[92, K, N])
    packed, scales = orc.quantize(W)
    X = inputs.activation(M, K, seed=[92, M, K])
    ws = w4.gemm_workspace(M, N, K, device="cuda")
    Y = w4.gemm_ws(dev(X), dev(packed.view(np.int32)), dev(scales.view(np.float16)),
                   ws).cpu().numpy()
    torch.cuda.synchronize()
    rows = np.random.default_rng([92, M]).choice(M, 24, replace=False)
    rows[:2] = (0, M - 1)
    check(Y, *orc.matmul(np.ascontiguousarray(X[rows]), packed, scales), rows=rows)


@pytest.mark.parametrize("M,K,N", [(128, 3584, 18944), (384, 4096, 14336), (128, 8192, 8192),
                                   (200, 8192, 8192)])
def test_prefill_split_wide_shapes_sampled(w4, orc, M, K, N):
    """K <= N shapes that the planner splits (slices of at least 10 groups
    that still fill the compute units): 3, 2, 7 and 4 K slices (24 sampled
    rows, the first and last included)."""
    say("prefill split wide M=%d K=%d N=%d" % (M, K, N))
    assert splits(w4, M, N, K)
    W = inputs.weight(N, K, seed=[95, K, N])
    packed, scales = orc.quantize(W)
    X = inputs.activation(M, K, seed=[95, M, K])
    ws = w4.gemm_workspace(M, N, K, device="cuda")
    Y = w4.gemm_ws(dev(X), dev(packed.view(np.int32)), dev(scales.view(np.float16)),
                   ws).cpu().numpy()
    torch.cuda.synchronize()
    rows = np.random.default_rng([95, M]).choice(M, 24, replace=False)
    rows[:2] = (0, M - 1)
    check(Y, *orc.matmul(np.ascontiguousarray(X[rows]), packed, scales), rows=rows)


def test_prefill_split_skips_short_slices(w4):
    """K <= N shapes whose split would give slices under 10 groups, or too
    few blocks, run unsplit (no workspace)."""
    for M, K, N in [(128, 4096, 14336), (128, 4096, 4096), (256, 4096, 4096), (512, 4096, 4096)]:
        assert not splits(w4, M, N, K), (M, K, N)


def test_prefill_split_workspace_reuse_and_determinism(w4, orc):
    """One workspace serves two shapes in a row (the second smaller);
    repeated calls give the same bits (fixed slice order); the unsplit
    w4a16_gemm meets the same bound."""
    shapes = [(300, 1000, 8192), (130, 600, 4096)]
    ws = w4.gemm_workspace(*shapes[0], device="cuda")
    for M, N, K in shapes:
        say("prefill split workspace M=%d N=%d K=%d" % (M, N, K))
        assert splits(w4, M, N, K)
        assert w4.library().w4a16_gemm_workspace_bytes(M, N, K) <= ws.numel()
        W = inputs.weight(N, K, seed=[93, N, K])
        packed, scales = orc.quantize(W)
        X = inputs.activation(M, K, seed=[93, M, K])
        pd, sd, Xd = dev(packed.view(np.int32)), dev(scales.view(np.float16)), dev(X)
        a = w4.gemm(Xd, pd, sd)
        b = w4.gemm_ws(Xd, pd, sd, ws)
        c = w4.gemm_ws(Xd, pd, sd, ws)
        torch.cuda.synchronize()
        assert torch.equal(b, c)
        ref = orc.matmul(X, packed, scales)
        check(b.cpu().numpy(), *ref)
        check(a.cpu().numpy(), *ref)


def test_prefill_split_graph_replays(w4, orc):
    """Captured in a graph: w4a16_gemm_ws (workspace) replays bit for bit as
    its eager call, beside an unsplit w4a16_gemm of the same shape."""
    M, N, K = 260, 1500, 6144
    assert splits(w4, M, N, K)
    W = inputs.weight(N, K, seed=[94])
    packed, scales = orc.quantize(W)
    X = inputs.activation(M, K, seed=[94, 1])
    pd, sd, Xd = dev(packed.view(np.int32)), dev(scales.view(np.float16)), dev(X)
    Yref, Yabs = orc.matmul(X, packed, scales)
    ws = w4.gemm_workspace(M, N, K, device="cuda")
    say("prefill split graph M=%d N=%d K=%d" % (M, N, K))
    eager = w4.gemm_ws(Xd, pd, sd, ws)
    torch.cuda.synchronize()
    out = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
    out2 = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        w4.gemm_ws(Xd, pd, sd, ws, Y=out)
        w4.gemm(Xd, pd, sd, Y=out2)
    for i in range(3):
        out.fill_(float("nan"))
        out2.fill_(float("nan"))
        junk = torch.randn(1 << 20, device="cuda").sum()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), "replay %d differs from eager" % i
        check(out2.cpu().numpy(), Yref, Yabs)
        del junk

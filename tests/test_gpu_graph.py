"""The library's launches captured in a HIP graph (as the benchmark does):
every replay, with eager work in between, equals the eager result."""
import numpy as np
import pytest

import oracle
from weight_only_int4_gemv_amd import inputs

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.mark.parametrize("M,algo", [(1, "gemv"), (4, "valu"), (16, "mfma"), (96, "mfma")])
def test_graph_replays_match_eager(M, algo):
    from weight_only_int4_gemv_amd import w4a16
    assert torch.cuda.is_available()
    N, K = 1536, 2304
    W, X = inputs.weight_and_activation(N, K, M, seed=[31, M])
    print("[case] graph %s M=%d" % (algo, M), flush=True)
    Wd, Xd = torch.from_numpy(W).cuda(), torch.from_numpy(X).cuda()
    packed, scales = w4a16.quantize(Wd)

    def call(out):
        if algo == "gemv":
            w4a16.gemv(Xd[0], packed, scales, y=out[0])
        else:
            w4a16.gemm(Xd, packed, scales, algo=algo, Y=out)

    eager = torch.empty((M, N), dtype=torch.float16, device="cuda")
    call(eager)
    torch.cuda.synchronize()
    out = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out)
    for i in range(4):
        out.fill_(float("nan"))
        junk = torch.randn(1 << 20, device="cuda").sum()          # eager work in between
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), "replay %d differs from eager" % i
        del junk
    po, so = oracle.get().quantize(W)
    yref, yabs = oracle.get().matmul(X, po, so)
    err = np.abs(out.cpu().numpy().astype(np.float64) - yref)
    assert (err <= oracle.tolerance(yref, yabs)).all()


@pytest.mark.parametrize("case", ["wide-prefill", "asym-tiled", "act-order", "4x4x4-k-split"])
def test_graph_replays_match_eager_more_paths(case):
    """The 128 x 256 prefill blocks (with their scale scan), the asymmetric
    tiled kernel, the act-order GEMV (x gathered through LDS) and the 4x4x4
    GEMV with two waves per row group (partial sums through LDS) under
    graph replay: every replay equals the eager result bit for bit."""
    from weight_only_int4_gemv_amd import w4a16
    assert torch.cuda.is_available()
    M, N, K = {"wide-prefill": (512, 8192, 1024), "asym-tiled": (96, 1536, 2304),
               "act-order": (1, 1536, 2304), "4x4x4-k-split": (4, 1536, 14336)}[case]
    W, X = inputs.weight_and_activation(N, K, M, seed=[33, M])
    print("[case] graph %s M=%d N=%d K=%d" % (case, M, N, K), flush=True)
    Wd, Xd = torch.from_numpy(W).cuda(), torch.from_numpy(X).cuda()
    if case == "asym-tiled":
        packed, scales, zeros = w4a16.quantize_asym(Wd)
    elif case == "act-order":
        perm = torch.from_numpy(np.random.default_rng(34).permutation(K).astype(np.int32)).cuda()
        packed, scales = w4a16.quantize(Wd, perm=perm)
    else:
        packed, scales = w4a16.quantize(Wd)

    def call(out):
        if case == "asym-tiled":
            w4a16.gemm_asym(Xd, packed, scales, zeros, Y=out)
        elif case == "act-order":
            w4a16.gemv(Xd[0], packed, scales, y=out[0], perm=perm)
        else:
            w4a16.gemm(Xd, packed, scales, algo="mfma", Y=out)

    eager = torch.empty((M, N), dtype=torch.float16, device="cuda")
    call(eager)
    torch.cuda.synchronize()
    assert torch.isfinite(eager).all()
    out = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out)
    for i in range(4):
        out.fill_(float("nan"))
        junk = torch.randn(1 << 20, device="cuda").sum()          # eager work in between
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), "replay %d differs from eager" % i
        del junk

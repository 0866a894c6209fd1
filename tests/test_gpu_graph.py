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

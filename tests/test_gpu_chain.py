"""w4a16_gemv_chain: a dependent sequence of decode GEMVs in one launch.

Its outputs must be bit-identical to separate w4a16_gemv calls (same
arithmetic and reduction order); a chain whose stages read the previous
stage's output checks the grid barrier (a stage that started early would
read a partial input and differ).  The sync buffer must come back zeroed.
"""
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


def say(msg):
    print("[case] " + msg, flush=True)


def make_weights(w4, shapes, seed):
    out = []
    for i, (K, N) in enumerate(shapes):
        W = inputs.weight(N, K, seed=[seed, i])
        p, s = w4.quantize(torch.from_numpy(W).cuda())
        out.append((K, N, p, s))
    return out


def run_dependent(w4, weights, x0, use_chain, sync=None):
    """x of stage s+1 is y of stage s."""
    ys = [torch.full((N,), float("nan"), dtype=torch.float16, device="cuda")
          for (_, N, _, _) in weights]
    xs = [x0] + ys[:-1]
    if use_chain:
        w4.gemv_chain([(xs[i], p, s, ys[i]) for i, (_, _, p, s) in enumerate(weights)], sync)
    else:
        for i, (_, _, p, s) in enumerate(weights):
            w4.gemv(xs[i], p, s, y=ys[i])
    torch.cuda.synchronize()
    return ys


@pytest.mark.parametrize("shapes", [
    [(1024, 2048), (2048, 3072), (3072, 1024), (1024, 4096), (4096, 640), (640, 300)],
    [(4096, 4096)] * 8,
    [(256, 256)] * 64,
    [(128, 128), (128, 3), (128, 128)],
    [(3584, 32768), (32768, 1536), (1536, 32770)],
], ids=["mixed", "square8", "small64", "tiny", "rows16"])
def test_chain_dependent_bit_identical(w4, shapes):
    # make every stage's K equal the previous N (data flows stage to stage)
    fixed = [shapes[0]]
    for K, N in shapes[1:]:
        fixed.append((fixed[-1][1] if fixed[-1][1] % 128 == 0 else K, N))
    chainable = all(fixed[i][0] == fixed[i - 1][1] for i in range(1, len(fixed)))
    if not chainable:
        fixed = [(K, N) for K, N in shapes]
    say("chain dependent %d stages %s" % (len(fixed), fixed[:3]))
    weights = make_weights(w4, fixed, seed=41)
    x0 = torch.from_numpy(inputs.activation(1, fixed[0][0], seed=42)[0]).cuda()
    sync = w4.chain_sync_buffer()
    if chainable:
        ref = run_dependent(w4, weights, x0, use_chain=False)
        got = run_dependent(w4, weights, x0, use_chain=True, sync=sync)
    else:
        xs = [torch.from_numpy(inputs.activation(1, K, seed=[43, i])[0]).cuda()
              for i, (K, _) in enumerate(fixed)]
        ref = [w4.gemv(xs[i], p, s) for i, (_, _, p, s) in enumerate(weights)]
        got = [torch.empty_like(r) for r in ref]
        w4.gemv_chain([(xs[i], p, s, got[i]) for i, (_, _, p, s) in enumerate(weights)], sync)
        torch.cuda.synchronize()
    for i, (a, b) in enumerate(zip(ref, got)):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), "stage %d differs" % i
    assert int(sync.abs().sum().item()) == 0, "sync buffer not returned to zero"


def test_chain_layer_shapes_against_oracle(w4):
    """One LLaMA-3-8B layer (qkv, o, gate_up, down) with synthetic inputs:
    every stage within the tolerance of the oracle."""
    orc = oracle.get()
    shapes = [(4096, 6144), (4096, 4096), (4096, 28672), (14336, 4096)]
    say("chain layer shapes")
    stages, refs = [], []
    for i, (K, N) in enumerate(shapes):
        W = inputs.weight(N, K, seed=[44, i])
        x = inputs.activation(1, K, seed=[45, i])
        po, so = orc.quantize(W)
        p = torch.from_numpy(po.view(np.int32)).cuda()
        s = torch.from_numpy(so.view(np.float16)).cuda()
        y = torch.empty((N,), dtype=torch.float16, device="cuda")
        stages.append((torch.from_numpy(x[0]).cuda(), p, s, y))
        refs.append(orc.matmul(x, po, so))
    sync = w4.chain_sync_buffer()
    w4.gemv_chain(stages, sync)
    torch.cuda.synchronize()
    for i, ((_, _, _, y), (yref, yabs)) in enumerate(zip(stages, refs)):
        err = np.abs(y.cpu().numpy().astype(np.float64) - yref[0])
        assert (err <= oracle.tolerance(yref[0], yabs[0])).all(), "stage %d" % i
        sep = w4.gemv(stages[i][0], stages[i][1], stages[i][2])
        assert torch.equal(sep.view(torch.int16), y.view(torch.int16))
    assert int(sync.abs().sum().item()) == 0


def test_chain_repeated_and_graph_replays(w4):
    shapes = [(2048, 2048)] * 5
    weights = make_weights(w4, shapes, seed=46)
    x0 = torch.from_numpy(inputs.activation(1, 2048, seed=47)[0]).cuda()
    sync = w4.chain_sync_buffer()
    say("chain repeated")
    ref = run_dependent(w4, weights, x0, use_chain=False)
    for _ in range(3):
        got = run_dependent(w4, weights, x0, use_chain=True, sync=sync)
        for a, b in zip(ref, got):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    say("chain graph")
    ys = [torch.empty((N,), dtype=torch.float16, device="cuda") for (_, N, _, _) in weights]
    xs = [x0] + ys[:-1]
    st = [(xs[i], p, s, ys[i]) for i, (_, _, p, s) in enumerate(weights)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        w4.gemv_chain(st, sync)
    for rep in range(4):
        for y in ys:
            y.fill_(float("nan"))
        junk = torch.randn(1 << 18, device="cuda").sum()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(ref, ys):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), "replay %d" % rep
        del junk
    assert int(sync.abs().sum().item()) == 0

"""w4a16_gemv_chain_noalloc: the dependent GEMV chain with the library's own
counter array instead of a caller buffer.

Checked against w4a16_gemv_chain (the entry point it is a variant of) on the
same stages: outputs bit-identical, on two calls in a row, the second with a
smaller input (fewer, smaller stages), then under graph replay.  The status
word reads 0 after every call (no wait gave up), which also shows the array
was left cleared by the call before.
"""
import pytest

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


def dependent_chain(w4, shapes, seed):
    """Weights for a chain where x of stage s+1 is y of stage s."""
    weights = []
    for i, (K, N) in enumerate(shapes):
        W = inputs.weight(N, K, seed=[seed, i])
        p, s = w4.quantize(torch.from_numpy(W).cuda())
        weights.append((K, N, p, s))
    x0 = torch.from_numpy(inputs.activation(1, shapes[0][0], seed=[seed, 99])[0]).cuda()
    return weights, x0


def stages_for(weights, x0):
    ys = [torch.full((N,), float("nan"), dtype=torch.float16, device="cuda")
          for (_, N, _, _) in weights]
    xs = [x0] + ys[:-1]
    return [(xs[i], p, s, ys[i]) for i, (_, _, p, s) in enumerate(weights)], ys


def reference(w4, weights, x0):
    st, ys = stages_for(weights, x0)
    sync = w4.chain_sync_buffer()
    w4.gemv_chain(st, sync)
    torch.cuda.synchronize()
    return ys


def same(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_noalloc_chain_matches_chain_two_calls(w4):
    big = [(1024, 2048), (2048, 3072), (3072, 1024), (1024, 4096), (4096, 640), (640, 1280)]
    small = [(512, 256), (256, 384), (384, 128)]
    status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    for name, shapes, seed in (("large", big, 71), ("smaller", small, 72)):
        say("noalloc chain, %s input: %d stages, first %s" % (name, len(shapes), shapes[0]))
        weights, x0 = dependent_chain(w4, shapes, seed)
        ref = reference(w4, weights, x0)
        st, ys = stages_for(weights, x0)
        status.fill_(-1)
        w4.gemv_chain_noalloc(st, status)
        torch.cuda.synchronize()
        assert int(status.item()) == 0, "a wait between stages gave up"
        for i, (a, b) in enumerate(zip(ref, ys)):
            assert same(a, b), "%s: stage %d differs from w4a16_gemv_chain" % (name, i)


def test_noalloc_chain_graph_replays(w4):
    shapes = [(2048, 2048)] * 4 + [(2048, 1024)]
    weights, x0 = dependent_chain(w4, shapes, 73)
    ref = reference(w4, weights, x0)
    st, ys = stages_for(weights, x0)
    status = torch.zeros((1,), dtype=torch.int32, device="cuda")
    say("noalloc chain graph capture")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        w4.gemv_chain_noalloc(st, status)
    for rep in range(4):
        for y in ys:
            y.fill_(float("nan"))
        status.fill_(-1)
        junk = torch.randn(1 << 18, device="cuda").sum()   # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert int(status.item()) == 0, "replay %d: a wait gave up" % rep
        for i, (a, b) in enumerate(zip(ref, ys)):
            assert same(a, b), "replay %d stage %d" % (rep, i)
        del junk


def test_noalloc_rejects_bad_arguments(w4):
    weights, x0 = dependent_chain(w4, [(128, 64)], 74)
    st, _ = stages_for(weights, x0)
    status = torch.zeros((1,), dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        w4.gemv_chain_noalloc(st * (w4.CHAIN_MAX + 1), status)
    lib = w4.library()
    arr = w4._chain_stages(st)
    assert lib.w4a16_gemv_chain_noalloc(arr, w4.CHAIN_MAX + 1, status.data_ptr(), None) == 1
    assert lib.w4a16_gemv_chain_noalloc(arr, 1, None, None) == 1
    assert lib.w4a16_gemv_chain_noalloc(arr, 1, status.data_ptr() + 2, None) == 3

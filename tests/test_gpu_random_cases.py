"""Seeded random cases across the options of the linear layer — group size
(32, 64, 128, 256, per channel), symmetric or asymmetric weights, act order,
kernel family (automatic, VALU, matrix cores), M from one token to a
512-token prompt, ragged N, K from 128 to 6144 — each against the oracle:
the GPU quantizer's bits where it takes the combination, and every output of
w4a16_linear within |y - y_ref| <= oracle.tolerance; and seeded long-K
shapes through w4a16_gemm_ws (K split over blocks where the planner splits)."""
import numpy as np
import pytest

import oracle
from weight_only_int4_gemv_amd import inputs

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

N_CASES = 144
MS = [1, 2, 3, 4, 5, 8, 13, 16, 17, 31, 32, 33, 64, 65, 100, 130, 257, 512]
GROUPS = [32, 64, 128, 256, -1]          # -1: one scale per row
ALGOS = [None, "valu", "mfma"]


def draw(i):
    rng = np.random.default_rng([20261203, i])
    group = GROUPS[int(rng.integers(len(GROUPS)))]
    unit = 256 if group == 256 else 128
    K = unit * int(rng.integers(1, 6144 // unit + 1))
    M = MS[int(rng.integers(len(MS)))]
    N = int(rng.integers(1, 3000))
    while M * N * K > 1.5e8 and N > 1:      # the oracle finishes in well under a second
        N //= 2
    return {"M": M, "N": N, "K": K, "group": group, "asym": bool(rng.random() < 0.4),
            "perm": bool(rng.random() < 0.3), "algo": ALGOS[int(rng.integers(len(ALGOS)))],
            "seed": [20261203, i]}


CASES = [draw(i) for i in range(N_CASES)]
IDS = ["%d-M%d-N%d-K%d-g%s%s%s-%s" % (i, c["M"], c["N"], c["K"],
                                       "pc" if c["group"] < 0 else c["group"],
                                       "-asym" if c["asym"] else "", "-perm" if c["perm"] else "",
                                       c["algo"] or "auto") for i, c in enumerate(CASES)]


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


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def test_cases_cover_every_option():
    """The draw reaches every group size, both weight kinds, act order, every
    kernel family, decode and prefill rows."""
    assert {c["group"] for c in CASES} == set(GROUPS)
    assert {c["asym"] for c in CASES} == {False, True}
    assert {c["perm"] for c in CASES} == {False, True}
    assert {c["algo"] for c in CASES} == set(ALGOS)
    assert min(c["M"] for c in CASES) <= 2 and max(c["M"] for c in CASES) >= 257


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_random_case(w4, orc, case):
    M, N, K, group = case["M"], case["N"], case["K"], case["group"]
    print("[case] %s" % IDS[CASES.index(case)], flush=True)
    og = K if group < 0 else group            # the oracle's group: the whole row
    W = (inputs.weight_skewed if case["asym"] else inputs.weight)(N, K, seed=case["seed"])
    X = inputs.activation(M, K, seed=[1000] + case["seed"])
    perm = (np.random.default_rng(case["seed"] + [1]).permutation(K).astype(np.int32)
            if case["perm"] else None)
    Wp = W if perm is None else np.ascontiguousarray(W[:, perm])
    if case["asym"]:
        packed, scales, zeros = orc.quantize_asym(Wp, group=og)
    else:
        (packed, scales), zeros = orc.quantize(Wp, group=og), None

    # the GPU quantizer (act order with symmetric weights only at group 128)
    Wd = dev(W)
    permd = dev(perm) if perm is not None else None
    got = None
    if case["asym"]:
        got = w4.quantize_asym(Wd, group=group, perm=permd)
        want = (packed, scales, zeros)
    elif perm is None or group == 128:
        got = w4.quantize(Wd, group=group, perm=permd)
        want = (packed, scales)
    if got is not None:
        torch.cuda.synchronize()
        for g, w_ in zip(got, want):
            g = g.cpu().numpy()
            assert np.array_equal(g.view(w_.dtype).reshape(w_.shape), w_), "quantizer bits differ"

    Y = w4.linear(dev(X), dev(packed.view(np.int32)), dev(scales.view(np.float16)),
                  dev(zeros) if zeros is not None else None, perm=permd, algo=case["algo"])
    Yg = Y.cpu().numpy().astype(np.float64)
    Xp = X if perm is None else np.ascontiguousarray(X[:, perm])
    if case["asym"]:
        Yref, Yabs = orc.matmul_asym(Xp, packed, scales, zeros, group=og)
    else:
        Yref, Yabs = orc.matmul(Xp, packed, scales, group=og)
    err = np.abs(Yg - Yref)
    bad = np.argwhere(~(err <= oracle.tolerance(Yref, Yabs)))
    assert bad.size == 0, "%d outputs out of tolerance, first %s: got %r want %r" % (
        len(bad), bad[0], Yg[tuple(bad[0])], Yref[tuple(bad[0])])


# K split over blocks through a workspace (w4a16_gemm_ws, group 128): long
# rows and few columns, where the planner splits K for batched decode (M <= 32)
# or for prefill (M > 64); shapes it does not split run as w4a16_gemm.
WS_MS = [5, 8, 13, 16, 24, 32, 65, 100, 200, 300, 512]


def draw_ws(i):
    rng = np.random.default_rng([20261204, i])
    K = 128 * int(rng.integers(16, 129))                 # 2048 .. 16384
    N = int(rng.integers(16, 4097))
    M = WS_MS[int(rng.integers(len(WS_MS)))]
    while M * N * K > 2e8 and N > 16:
        N //= 2
    return {"M": M, "N": N, "K": K, "seed": [20261204, i]}


WS_CASES = [draw_ws(i) for i in range(24)]


def test_ws_cases_reach_both_splits(w4):
    """The long-K draw includes shapes the planner splits for batched decode
    (M <= 32) and for prefill (M > 64), and shapes it leaves unsplit."""
    split = [(c["M"], w4.gemm_workspace(c["M"], c["N"], c["K"]).numel() > 1) for c in WS_CASES]
    assert any(s for m, s in split if m <= 32) and any(s for m, s in split if m > 64)
    assert not all(s for _, s in split)


@pytest.mark.parametrize("case", WS_CASES,
                         ids=["%d-M%d-N%d-K%d" % (i, c["M"], c["N"], c["K"])
                              for i, c in enumerate(WS_CASES)])
def test_random_ws_case(w4, orc, case):
    M, N, K = case["M"], case["N"], case["K"]
    print("[ws case] M=%d N=%d K=%d" % (M, N, K), flush=True)
    W = inputs.weight(N, K, seed=case["seed"])
    X = inputs.activation(M, K, seed=[1000] + case["seed"])
    packed, scales = orc.quantize(W)
    ws = w4.gemm_workspace(M, N, K)
    Yd = torch.empty((M, N), dtype=torch.float16, device="cuda")
    w4.gemm_ws(dev(X), dev(packed.view(np.int32)), dev(scales.view(np.float16)), ws, Yd)
    Yg = Yd.cpu().numpy().astype(np.float64)
    Yref, Yabs = orc.matmul(X, packed, scales)
    bad = np.argwhere(~(np.abs(Yg - Yref) <= oracle.tolerance(Yref, Yabs)))
    assert bad.size == 0, "%d outputs out of tolerance, first %s: got %r want %r" % (
        len(bad), bad[0], Yg[tuple(bad[0])], Yref[tuple(bad[0])])

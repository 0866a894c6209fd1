"""M = 1 GEMV on rows of K/32 = 16, 48 or 112 chunks with at least 128 rows
per compute unit, where the persistent kernel holds four rows side by side
per register slot (16 lanes each, the row offset in the lane offset and the
slot's in the scalar offset): every weight variant on that layout — act
order, asymmetric INT4, both, group sizes 32 / 64 / 128 / 256 and one scale
per row — against the oracle, ragged N (a last row group of three rows)."""
import numpy as np
import pytest

import oracle
from weight_only_int4_gemv_amd import inputs

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

# (K, group, asymmetric, act order); group -1: one scale per row
CASES = [(512, 128, False, True), (1536, 32, False, True), (3584, 64, False, False),
         (3584, 128, True, False), (1536, 64, True, True), (512, 256, True, False),
         (1536, -1, False, False), (3584, -1, True, True), (3584, 256, False, True)]
IDS = ["K%d-g%s%s%s" % (K, "pc" if g < 0 else g, "-asym" if a else "", "-perm" if p else "")
       for K, g, a, p in CASES]


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


@pytest.mark.parametrize("K,group,asym,perm", CASES, ids=IDS)
def test_gemv_four_rows_per_slot(w4, orc, K, group, asym, perm):
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    N = 128 * ncu + 3
    seed = [77, K, K if group < 0 else group, int(asym), int(perm)]
    print("[rows16] N=%d K=%d group=%d asym=%s perm=%s" % (N, K, group, asym, perm), flush=True)
    og = K if group < 0 else group
    W = (inputs.weight_skewed if asym else inputs.weight)(N, K, seed=seed)
    x = inputs.activation(1, K, seed=[1000] + seed)
    p = np.random.default_rng(seed + [1]).permutation(K).astype(np.int32) if perm else None
    Wp = W if p is None else np.ascontiguousarray(W[:, p])
    if asym:
        packed, scales, zeros = orc.quantize_asym(Wp, group=og)
    else:
        (packed, scales), zeros = orc.quantize(Wp, group=og), None
    Y = w4.linear(dev(x), dev(packed.view(np.int32)), dev(scales.view(np.float16)),
                  dev(zeros) if zeros is not None else None,
                  perm=dev(p) if p is not None else None)
    Yg = Y.cpu().numpy().astype(np.float64)
    xp = x if p is None else np.ascontiguousarray(x[:, p])
    if asym:
        Yref, Yabs = orc.matmul_asym(xp, packed, scales, zeros, group=og)
    else:
        Yref, Yabs = orc.matmul(xp, packed, scales, group=og)
    bad = np.argwhere(~(np.abs(Yg - Yref) <= oracle.tolerance(Yref, Yabs)))
    assert bad.size == 0, "%d outputs out of tolerance, first %s: got %r want %r" % (
        len(bad), bad[0], Yg[tuple(bad[0])], Yref[tuple(bad[0])])

"""C ABI on the host: the library loads, exports every declared symbol, and
validates arguments before touching a device (no kernel is launched here)."""
import ctypes
import os
import re
import subprocess

import pytest

from weight_only_int4_gemv_amd import w4a16

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4a16.h")

OK, INVALID, SHAPE, MISALIGNED, DEVICE = 0, 1, 2, 3, 4
FAKE = 0x10000  # 64 KiB-aligned host address; only ever rejected before use


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*[\w\s\*]+?\b(w4a16_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(w4a16.LIBRARY):
        from weight_only_int4_gemv_amd import build
        build.build()
    return w4a16.library()


def test_header_declares_the_boundary():
    names = declared_functions()
    for fn in ["w4a16_quantize", "w4a16_gemv", "w4a16_gemm", "w4a16_gemm_ex",
               "w4a16_packed_bytes", "w4a16_scales_bytes", "w4a16_status_string",
               "w4a16_valu_max_m", "w4a16_quantize_g", "w4a16_gemv_g", "w4a16_gemm_g",
               "w4a16_scales_bytes_g", "w4a16_quantize_perm", "w4a16_gemv_perm",
               "w4a16_gemm_perm", "w4a16_quantize_asym", "w4a16_gemv_asym",
               "w4a16_gemm_asym", "w4a16_q4_0_bytes", "w4a16_quantize_q4_0",
               "w4a16_gemv_q4_0", "w4a16_gemm_q4_0", "w4a16_gemv_chain",
               "w4a16_gemv_chain_noalloc", "w4a16_gemm_ws", "w4a16_gemm_workspace_bytes",
               "w4a16_linear", "w4a16_linear_workspace_bytes", "w4a16_gemm_asym_ws",
               "w4a16_gemm_asym_workspace_bytes"]:
        assert fn in names


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", w4a16.LIBRARY], check=True,
                         capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (w4a16_\w+)$", out, re.M))
    for fn in declared_functions():
        assert fn in exported, fn
        assert hasattr(lib, fn)


def test_no_torch_types_in_header():
    text = open(HEADER).read()
    assert "torch" not in text and "at::" not in text and "hip_runtime" not in text


def test_size_helpers(lib):
    assert lib.w4a16_packed_bytes(4096, 4096) == 4096 * 4096 // 2
    assert lib.w4a16_scales_bytes(4096, 4096) == 4096 * 32 * 2
    assert lib.w4a16_packed_bytes(14336, 4096) * 2 == 4096 * 14336
    # 2 bytes of scale per 64 bytes of codes: 3.125 %
    assert lib.w4a16_scales_bytes(512, 1024) * 32 == lib.w4a16_packed_bytes(512, 1024)
    assert lib.w4a16_packed_bytes(4, 100) == 0       # K % 128 != 0
    assert lib.w4a16_packed_bytes(-1, 128) == 0
    assert lib.w4a16_scales_bytes(4, -128) == 0


def test_status_strings(lib):
    for st in range(6):
        assert len(w4a16.status_string(st)) >= 2
    assert w4a16.status_string(99) == "unknown status"


def test_quantize_validation(lib):
    q = lib.w4a16_quantize
    assert q(FAKE, 4, 100, FAKE, FAKE, None) == SHAPE
    assert q(FAKE, -4, 128, FAKE, FAKE, None) == INVALID
    assert q(FAKE, 4, 1 << 31, FAKE, FAKE, None) == INVALID
    assert q(FAKE, (1 << 24) + 1, 128, FAKE, FAKE, None) == INVALID
    assert q(None, 4, 128, FAKE, FAKE, None) == INVALID
    assert q(FAKE, 4, 128, None, FAKE, None) == INVALID
    assert q(FAKE, 4, 128, FAKE, None, None) == INVALID
    assert q(FAKE + 8, 4, 128, FAKE * 2, FAKE * 3, None) == MISALIGNED
    assert q(FAKE, 4, 128, FAKE * 2 + 4, FAKE * 3, None) == MISALIGNED
    assert q(FAKE, 4, 128, FAKE * 2, FAKE * 3 + 1, None) == MISALIGNED
    # outputs overlapping the input or each other
    assert q(FAKE, 4, 128, FAKE + 256, FAKE * 3, None) == INVALID
    assert q(FAKE, 4, 128, FAKE * 2, FAKE * 2 + 32, None) == INVALID
    # empty problems enqueue nothing and accept NULL
    assert q(None, 0, 128, None, None, None) == OK
    assert q(None, 5, 0, None, None, None) == OK


def test_linear_validation(lib):
    g = lib.w4a16_gemm_ex
    A, B, C, D = FAKE, FAKE * 4, FAKE * 8, FAKE * 12
    assert g(A, 2, B, C, 16, 100, D, 0, None) == SHAPE
    assert g(A, -2, B, C, 16, 128, D, 0, None) == INVALID
    assert g(A, 2, B, C, -16, 128, D, 0, None) == INVALID
    assert g(A, 2, B, C, 16, 128, D, 7, None) == INVALID        # unknown algo
    assert g(A, (1 << 24) + 1, B, C, 16, 128, D, 0, None) == INVALID
    assert g(A, 2, B, C, (1 << 24) + 1, 128, D, 0, None) == INVALID
    assert g(None, 2, B, C, 16, 128, D, 0, None) == INVALID
    assert g(A, 2, None, C, 16, 128, D, 0, None) == INVALID
    assert g(A, 2, B, None, 16, 128, D, 0, None) == INVALID
    assert g(A, 2, B, C, 16, 128, None, 0, None) == INVALID
    assert g(A + 2, 2, B, C, 16, 128, D, 0, None) == MISALIGNED
    assert g(A, 2, B + 4, C, 16, 128, D, 0, None) == MISALIGNED
    assert g(A, 2, B, C + 1, 16, 128, D, 0, None) == MISALIGNED
    assert g(A, 2, B, C, 16, 128, D + 1, 0, None) == MISALIGNED
    assert g(A, 2, B, C, 16, 128, A + 16, 0, None) == INVALID   # Y overlaps X
    assert g(A, 2, B, C, 16, 128, B, 0, None) == INVALID        # Y overlaps packed
    assert g(A, 2, B, C, 16, 128, C + 2, 0, None) == INVALID    # Y overlaps scales
    assert g(None, 0, None, None, 16, 128, None, 0, None) == OK
    assert g(None, 3, None, None, 0, 128, None, 0, None) == OK
    gv = lib.w4a16_gemv
    assert gv(A, B, C, 16, 130, D, None) == SHAPE
    assert gv(A + 8, B, C, 16, 128, D, None) == MISALIGNED
    assert gv(A, B, C, 0, 128, None, None) == OK


def test_group_size_validation(lib):
    """Group size as a parameter: 32, 64, 128, 256 accepted, anything else is an
    invalid argument; K must be a multiple of the group; scale bytes follow
    N*(K/group)*2."""
    sb = lib.w4a16_scales_bytes_g
    assert sb(4096, 4096, 32) == 4096 * 128 * 2
    assert sb(4096, 4096, 64) == 4096 * 64 * 2
    assert sb(4096, 4096, 128) == lib.w4a16_scales_bytes(4096, 4096)
    assert sb(4096, 4096, 256) == 4096 * 16 * 2
    assert sb(4, 384, 256) == 0        # 384 % 256 != 0
    assert sb(4, 128, 48) == 0 and sb(4, 128, 16) == 0 and sb(4, 128, 512) == 0
    q = lib.w4a16_quantize_g
    assert q(FAKE, 4, 128, 16, FAKE * 2, FAKE * 3, None) == INVALID
    assert q(FAKE, 4, 128, 96, FAKE * 2, FAKE * 3, None) == INVALID
    assert q(FAKE, 4, 384, 256, FAKE * 2, FAKE * 3, None) == SHAPE
    assert q(FAKE, 4, 100, 32, FAKE * 2, FAKE * 3, None) == SHAPE
    # scales of 4 x 128 at group 32 take 32 bytes: placed 24 bytes before
    # packed they overlap it, at group 128 (8 bytes) they would not
    assert q(FAKE, 4, 128, 32, FAKE * 2, FAKE * 2 - 24, None) == INVALID
    assert lib.w4a16_scales_bytes_g(4, 128, 128) == 8
    assert q(None, 0, 256, 256, None, None, None) == OK
    A, B, C, D = FAKE, FAKE * 4, FAKE * 8, FAKE * 12
    gv, gm = lib.w4a16_gemv_g, lib.w4a16_gemm_g
    assert gv(A, B, C, 16, 128, 100, D, None) == INVALID
    assert gv(A, B, C, 16, 384, 256, D, None) == SHAPE
    assert gm(A, 2, B, C, 16, 128, 0, D, None) == INVALID
    # Y 40 bytes after the scales: inside their 128 bytes at group 32
    # (16 rows x 4 groups), past their 32 bytes at group 128
    assert gm(A, 2, B, C, 16, 128, 32, C + 40, None) == INVALID
    assert gm(None, 0, None, None, 16, 256, 256, None, None) == OK
    # the binding infers the group from the scales' shape and checks it
    import torch
    with pytest.raises(ValueError):
        w4a16.quantize(torch.zeros(4, 128, dtype=torch.float16), group=48)
    with pytest.raises(ValueError):
        w4a16.gemv(torch.zeros(256, dtype=torch.float16),
                   torch.zeros(4, 32, dtype=torch.int32),
                   torch.zeros(4, 3, dtype=torch.float16))       # 256 / 3: no group


def test_act_order_validation(lib):
    """Act-order entry points: perm is required for K > 0, 16-byte aligned,
    and no output may overlap it."""
    A, B, C, D, P = FAKE, FAKE * 4, FAKE * 8, FAKE * 12, FAKE * 16
    q, gv, gm = lib.w4a16_quantize_perm, lib.w4a16_gemv_perm, lib.w4a16_gemm_perm
    assert q(A, None, 4, 128, B, C, None) == INVALID
    assert q(A, P + 4, 4, 128, B, C, None) == MISALIGNED
    assert q(A, B + 64, 4, 128, B, C, None) == INVALID        # packed overlaps perm
    assert q(A, P, 4, 100, B, C, None) == SHAPE
    assert q(None, None, 0, 128, None, None, None) == OK
    assert gv(A, None, B, C, 16, 128, D, None) == INVALID
    assert gv(A, P + 8, B, C, 16, 128, D, None) == MISALIGNED
    assert gv(A, P, B, C, 16, 128, P + 2, None) == INVALID      # y overlaps perm
    assert gm(A, 2, None, B, C, 16, 128, D, None) == INVALID
    assert gm(A, 2, P, B, C, 16, 130, D, None) == SHAPE
    assert gm(None, 0, None, None, None, 16, 128, None, None) == OK
    import torch
    with pytest.raises(ValueError):
        w4a16.gemv(torch.zeros(128, dtype=torch.float16),
                   torch.zeros(4, 16, dtype=torch.int32), torch.zeros(4, 1, dtype=torch.float16),
                   perm=torch.zeros(128, dtype=torch.int64))


def test_asymmetric_validation(lib):
    """Asymmetric entry points: zeros required for K > 0 and 2-byte aligned,
    perm optional, no output overlapping another output or an input, group
    checked as for the group-size entry points."""
    A, B, C, D, P, Z = FAKE, FAKE * 4, FAKE * 8, FAKE * 12, FAKE * 16, FAKE * 20
    q, gv, gm = lib.w4a16_quantize_asym, lib.w4a16_gemv_asym, lib.w4a16_gemm_asym
    assert q(A, None, 4, 128, 128, B, C, None, None) == INVALID        # no zeros
    assert q(A, None, 4, 128, 128, B, C, Z + 1, None) == MISALIGNED
    assert q(A, None, 4, 128, 128, B, C, C + 4, None) == INVALID       # zeros overlap scales
    assert q(A, None, 4, 128, 128, B, C, B + 8, None) == INVALID       # zeros overlap packed
    assert q(A, None, 4, 128, 128, B, C, A + 16, None) == INVALID      # zeros overlap W
    assert q(A, P, 4, 128, 128, B, C, P + 16, None) == INVALID         # zeros overlap perm
    assert q(A, P + 4, 4, 128, 128, B, C, Z, None) == MISALIGNED
    assert q(A, None, 4, 128, 48, B, C, Z, None) == INVALID            # group
    assert q(A, None, 4, 192, 128, B, C, Z, None) == SHAPE
    assert q(A, None, 4, 384, 256, B, C, Z, None) == SHAPE
    assert q(None, None, 0, 128, 128, None, None, None, None) == OK
    assert gv(A, None, B, C, None, 16, 128, 128, D, None) == INVALID   # no zeros
    assert gv(A, None, B, C, Z + 1, 16, 128, 128, D, None) == MISALIGNED
    assert gv(A, None, B, C, Z, 16, 128, 128, Z + 2, None) == INVALID  # y overlaps zeros
    assert gv(A, P, B, C, Z, 16, 128, 128, P + 2, None) == INVALID     # y overlaps perm
    assert gv(A, None, B, C, Z, 16, 128, 64 + 1, D, None) == INVALID
    assert gm(A, 2, None, B, C, None, 16, 128, 128, D, None) == INVALID
    assert gm(A, 2, None, B, C, Z, 16, 130, 128, D, None) == SHAPE
    assert gm(A, -1, None, B, C, Z, 16, 128, 128, D, None) == INVALID
    assert gm(None, 0, None, None, None, None, 16, 128, 128, None, None) == OK
    import torch
    with pytest.raises(ValueError):
        w4a16.quantize_asym(torch.zeros(4, 128, dtype=torch.float16), group=48)
    with pytest.raises(ValueError):
        w4a16.gemv_asym(torch.zeros(128, dtype=torch.float16),
                        torch.zeros(4, 16, dtype=torch.int32),
                        torch.zeros(4, 1, dtype=torch.float16),
                        torch.zeros(4, 1, dtype=torch.int32))       # zeros must be int16


def test_q4_0_validation(lib):
    """Q4_0 entry points: sizes (18 bytes per 32 elements), alignment,
    overlap, the K limit of the staged-activation GEMV."""
    A, B, D = FAKE, FAKE * 4, FAKE * 12
    assert lib.w4a16_q4_0_bytes(4096, 4096) == 4096 * 128 * 18
    assert lib.w4a16_q4_0_bytes(1, 128) == 80                        # 72 rounded up to 16
    assert lib.w4a16_q4_0_bytes(3, 100) == 0 and lib.w4a16_q4_0_bytes(-1, 128) == 0
    q, gv, gm = lib.w4a16_quantize_q4_0, lib.w4a16_gemv_q4_0, lib.w4a16_gemm_q4_0
    assert q(A, 4, 100, B, None) == SHAPE
    assert q(A, 4, 128, None, None) == INVALID
    assert q(A, 4, 128, B + 2, None) == MISALIGNED
    assert q(A, 4, 128, A + 64, None) == INVALID                     # blocks overlap W
    assert q(None, 0, 128, None, None) == OK
    assert gv(A, B, 16, 128, None, None) == INVALID
    assert gv(A, B + 8, 16, 128, D, None) == MISALIGNED
    assert gv(A, B, 16, 128, B + 2, None) == INVALID                 # y overlaps blocks
    assert gv(A, B, 16, 32768 + 128, D, None) == INVALID             # K beyond the LDS budget
    assert gv(A, B, 16, 200, D, None) == SHAPE
    assert gm(A, -1, B, 16, 128, D, None) == INVALID
    assert gm(None, 0, None, 16, 128, None, None) == OK
    import torch
    with pytest.raises(ValueError):
        w4a16.gemv_q4_0(torch.zeros(128, dtype=torch.float16),
                        torch.zeros(4, 70, dtype=torch.uint8))       # not whole blocks


@pytest.mark.skipif(__import__("torch").cuda.device_count() > 0,
                    reason="with a GPU present valid arguments would launch")
def test_valid_arguments_without_device_report_device_error(lib):
    A, B, C, D = FAKE, FAKE * 4, FAKE * 8, FAKE * 12
    assert lib.w4a16_gemm(A, 2, B, C, 16, 128, D, None) == DEVICE
    assert lib.w4a16_quantize(A, 4, 128, B, C, None) == DEVICE
    assert lib.w4a16_quantize_g(A, 4, 256, 64, B, C, None) == DEVICE
    assert lib.w4a16_gemm_g(A, 2, B, C, 16, 256, 256, D, None) == DEVICE
    assert lib.w4a16_gemv_perm(A, FAKE * 16, B, C, 16, 128, D, None) == DEVICE
    assert lib.w4a16_quantize_asym(A, None, 4, 128, 128, B, C, FAKE * 20, None) == DEVICE
    assert lib.w4a16_gemm_asym(A, 2, None, B, C, FAKE * 20, 16, 128, 64, D, None) == DEVICE
    assert lib.w4a16_quantize_q4_0(A, 4, 128, B, None) == DEVICE
    assert lib.w4a16_gemm_q4_0(A, 3, B, 16, 256, D, None) == DEVICE


def test_binding_rejects_bad_tensors():
    import torch
    W = torch.zeros(4, 128, dtype=torch.float16)          # on the CPU
    with pytest.raises(ValueError):
        w4a16.quantize(W)
    with pytest.raises(ValueError):
        w4a16.gemv(torch.zeros(128, dtype=torch.float16),
                   torch.zeros(4, 16, dtype=torch.int32),
                   torch.zeros(4, 1, dtype=torch.float16))
    with pytest.raises(ValueError):
        w4a16.gemm(torch.zeros(2, 128, dtype=torch.float32),
                   torch.zeros(4, 16, dtype=torch.int32),
                   torch.zeros(4, 1, dtype=torch.float16))


def test_chain_validation(lib):
    from weight_only_int4_gemv_amd.w4a16 import GemvStage
    A, B, C, D, S = FAKE, FAKE * 4, FAKE * 8, FAKE * 12, FAKE * 16
    ch = lib.w4a16_gemv_chain

    def arr(*stages):
        a = (GemvStage * len(stages))()
        for i, s in enumerate(stages):
            a[i] = s
        return a
    ok = GemvStage(A, B, C, D, 16, 128)
    assert ch(arr(ok), 0, S, None) == OK                      # empty: nothing enqueued
    assert ch(arr(ok), -1, S, None) == INVALID
    assert ch(arr(ok), 65, S, None) == INVALID
    assert ch(arr(ok), 1, None, None) == INVALID
    assert ch(arr(ok), 1, S + 2, None) == MISALIGNED
    assert ch(arr(GemvStage(A, B, C, D, 16, 100)), 1, S, None) == SHAPE
    assert ch(arr(GemvStage(A, B, C, D, 16, 0)), 1, S, None) == SHAPE
    assert ch(arr(GemvStage(A, B, C, D, 16, 32768 + 128)), 1, S, None) == INVALID
    assert ch(arr(GemvStage(A, B, C, D, 0, 128)), 1, S, None) == INVALID
    assert ch(arr(GemvStage(A, B, C, D, (1 << 20) + 1, 128)), 1, S, None) == INVALID
    assert ch(arr(GemvStage(A + 8, B, C, D, 16, 128)), 1, S, None) == MISALIGNED
    assert ch(arr(GemvStage(A, B, C, A + 64, 16, 128)), 1, S, None) == INVALID   # y on own x
    assert ch(arr(GemvStage(A, B, C, B, 16, 128)), 1, S, None) == INVALID       # y on packed
    assert ch(arr(GemvStage(A, B, C, D, 16, 128), GemvStage(A, B + 1024, D, D + 256, 16, 128)),
              2, S, None) == INVALID                                           # y on scales
    assert ch(arr(GemvStage(A, B, C, D, 16, 128)), 1, D, None) == INVALID      # sync on y


def test_chain_noalloc_validation(lib):
    """The no-allocation chain validates like w4a16_gemv_chain, plus its status
    word (required, 4-byte aligned, not on any stage tensor)."""
    from weight_only_int4_gemv_amd.w4a16 import GemvStage
    A, B, C, D, S = FAKE, FAKE * 4, FAKE * 8, FAKE * 12, FAKE * 16
    ch = lib.w4a16_gemv_chain_noalloc
    a = (GemvStage * 1)()
    a[0] = GemvStage(A, B, C, D, 16, 128)
    assert ch(a, 0, S, None) == OK                       # empty: nothing enqueued
    assert ch(a, -1, S, None) == INVALID
    assert ch(a, 65, S, None) == INVALID                 # beyond the counters' stage limit
    assert ch(a, 1, None, None) == INVALID               # status is required
    assert ch(a, 1, S + 2, None) == MISALIGNED
    assert ch(a, 1, D, None) == INVALID                  # status on an output
    assert ch(a, 1, B + 64, None) == INVALID             # status on the weights
    b = (GemvStage * 1)()
    b[0] = GemvStage(A, B, C, D, 16, 100)
    assert ch(b, 1, S, None) == SHAPE
    assert ch(a, 1, S, None) in (DEVICE, OK)             # valid: only the device is left


def test_gemm_ws_validation(lib):
    """Sizes are checked before the device; the split plan (and so the
    workspace size) needs a gfx950 device, so without one the size is 0 and
    valid calls report the device error."""
    A, B, C, D, S = FAKE, FAKE * 4, FAKE * 8, FAKE * 12, FAKE * 16
    f = lib.w4a16_gemm_ws
    n = lib.w4a16_gemm_workspace_bytes(16, 4096, 14336)
    assert n == 0 or n > 4096          # 0 without a gfx950 device
    assert lib.w4a16_gemm_workspace_bytes(-1, 4096, 14336) == 0
    assert lib.w4a16_gemm_workspace_bytes(16, 4096, 100) == 0
    assert f(A, -1, B, C, 16, 128, D, S, 4096, None) == INVALID
    assert f(A, 4, B, C, 16, 100, D, S, 4096, None) == SHAPE
    assert f(A, 0, B, C, 16, 128, D, S, 4096, None) == OK      # empty: nothing enqueued
    assert f(None, 4, B, C, 16, 128, D, S, 4096, None) == INVALID
    assert f(A, 4, B, C, 16, 128, D, S, 4096, None) in (DEVICE, OK)


def test_gemm_asym_ws_validation(lib):
    """The asymmetric K split: sizes and the group are checked before the
    device; without a gfx950 device the workspace size is 0 and valid calls
    report the device error."""
    A, B, C, Z, D, S = FAKE, FAKE * 4, FAKE * 8, FAKE * 10, FAKE * 12, FAKE * 16
    f = lib.w4a16_gemm_asym_ws
    n = lib.w4a16_gemm_asym_workspace_bytes(128, 4096, 14336, 128)
    assert n == 0 or n > 4096          # 0 without a gfx950 device
    assert lib.w4a16_gemm_asym_workspace_bytes(-1, 4096, 14336, 128) == 0
    assert lib.w4a16_gemm_asym_workspace_bytes(128, 4096, 100, 128) == 0
    assert lib.w4a16_gemm_asym_workspace_bytes(128, 4096, 14336, 64) == 0   # group 128 only
    assert lib.w4a16_gemm_asym_workspace_bytes(128, 4096, 14336, 48) == 0   # no such group
    assert f(A, -1, B, C, Z, 16, 128, 128, D, S, 4096, None) == INVALID
    assert f(A, 4, B, C, Z, 16, 100, 128, D, S, 4096, None) == SHAPE        # K not a multiple of 128
    assert f(A, 4, B, C, Z, 16, 128, 48, D, S, 4096, None) == INVALID       # unknown group
    assert f(A, 0, B, C, Z, 16, 128, 128, D, S, 4096, None) == OK           # empty: nothing enqueued
    assert f(A, 4, B, C, None, 16, 128, 128, D, S, 4096, None) == INVALID   # zeros required
    assert f(A, 4, B, C, Z, 16, 128, 128, D, S, 4096, None) in (DEVICE, OK)


def test_linear_general_validation(lib):
    """w4a16_linear: every option of the linear layer in one call; the
    act-order workspace is checked (size, alignment, overlap with every
    operand) before the device; NULL perm and zeros mean none."""
    A, B, C, D, P, Z, W = (FAKE, FAKE * 4, FAKE * 8, FAKE * 12, FAKE * 16, FAKE * 20,
                           FAKE * 64)
    f = lib.w4a16_linear
    wb = lib.w4a16_linear_workspace_bytes
    assert wb(512, 4096, 1) == 512 * 4096 * 2
    assert wb(512, 4096, 0) == 0
    assert wb(-1, 4096, 1) == 0 and wb(4, 100, 1) == 0
    need = wb(4, 256, 1)
    # sizes, group, algo
    assert f(A, -1, None, B, C, None, 16, 256, 128, D, 0, None, 0, None) == INVALID
    assert f(A, 4, None, B, C, None, 16, 200, 128, D, 0, None, 0, None) == SHAPE
    assert f(A, 4, None, B, C, None, 16, 256, 48, D, 0, None, 0, None) == INVALID
    assert f(A, 4, None, B, C, None, 16, 384, 256, D, 0, None, 0, None) == SHAPE
    assert f(A, 4, None, B, C, None, 16, 256, 128, D, 9, None, 0, None) == INVALID
    # misaligned or overlapping operands as for the other forms
    assert f(A, 4, P + 4, B, C, None, 16, 256, 128, D, 0, None, 0, None) == MISALIGNED
    assert f(A, 4, None, B, C, Z + 1, 16, 256, 128, D, 0, None, 0, None) == MISALIGNED
    assert f(A, 4, P, B, C, None, 16, 256, 128, P + 2, 0, None, 0, None) == INVALID
    assert f(A, 4, None, B, C, Z, 16, 256, 128, Z + 2, 0, None, 0, None) == INVALID
    # workspace: too small, misaligned, overlapping X, Y, packed, scales, perm, zeros
    assert f(A, 4, P, B, C, None, 16, 256, 128, D, 2, W, need - 1, None) == INVALID
    assert f(A, 4, P, B, C, None, 16, 256, 128, D, 2, W + 8, need, None) == MISALIGNED
    assert f(A, 4, P, B, C, None, 16, 256, 128, D, 2, A + 16, need, None) == INVALID
    assert f(A, 4, P, B, C, None, 16, 256, 128, D, 2, D - 16, need, None) == INVALID
    assert f(A, 4, P, B, C, None, 16, 256, 128, D, 2, B + 16, need, None) == INVALID
    assert f(A, 4, P, B, C, None, 16, 256, 128, D, 2, C - 16, need, None) == INVALID
    assert f(A, 4, P, B, C, None, 16, 256, 128, D, 2, P - 16, need, None) == INVALID
    assert f(A, 4, P, B, C, Z, 16, 256, 128, D, 2, Z - 16, need, None) == INVALID
    # without a perm the workspace is not used and not checked
    assert f(A, 4, None, B, C, None, 16, 256, 128, D, 2, W + 8, 0, None) in (DEVICE, OK)
    # valid calls reach the device check
    assert f(A, 4, P, B, C, Z, 16, 256, 32, D, 2, W, need, None) in (DEVICE, OK)
    assert f(A, 4, P, B, C, None, 16, 256, -1, D, 0, None, 0, None) in (DEVICE, OK)
    assert f(None, 0, None, None, None, None, 16, 256, 128, None, 0, None, 0, None) == OK

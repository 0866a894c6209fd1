"""Python binding of ``libw4a16.so`` (the C ABI in include/w4a16.h).

Argument marshalling only: torch supplies device memory and the current
stream; every step of the computation runs in the library's HIP kernels.
There is no fallback: a missing library or a non-gfx950 device is an error.

    packed, scales = quantize(W)            # W: fp16 [N, K] on the GPU
    y = gemv(x, packed, scales)             # x: fp16 [K]      -> [N]
    Y = gemm(X, packed, scales)             # X: fp16 [M, K]   -> [M, N]
    packed, scales, zeros = quantize_asym(W)          # asymmetric INT4
    Y = gemm_asym(X, packed, scales, zeros)
"""
from __future__ import annotations

import ctypes
import os

import torch

LIBRARY = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libw4a16.so")

W4A16_GROUP = 128
ALGO_AUTO, ALGO_VALU, ALGO_MFMA = 0, 1, 2
_ALGOS = {None: ALGO_AUTO, "auto": ALGO_AUTO, "valu": ALGO_VALU, "mfma": ALGO_MFMA}

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_lib = None


CHAIN_MAX = 64
CHAIN_SYNC_WORDS = 1024
CHAIN_ERR_WORD = 0


class GemvStage(ctypes.Structure):
    """w4a16_gemv_stage of include/w4a16.h."""
    _fields_ = [("x", _p), ("packed", _p), ("scales", _p), ("y", _p),
                ("N", _i64), ("K", _i64)]


class W4A16Error(RuntimeError):
    """A non-zero status from the library."""

    def __init__(self, fn: str, status: int):
        super().__init__("%s failed: status %d (%s)" % (fn, status, status_string(status)))
        self.status = status


def library() -> ctypes.CDLL:
    """The loaded library (loaded on first use; raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIBRARY):
            raise ImportError("%s is not built: run python -m weight_only_int4_gemv_amd.build"
                              % LIBRARY)
        lib = ctypes.CDLL(LIBRARY)
        lib.w4a16_packed_bytes.argtypes = [_i64, _i64]
        lib.w4a16_packed_bytes.restype = ctypes.c_size_t
        lib.w4a16_scales_bytes.argtypes = [_i64, _i64]
        lib.w4a16_scales_bytes.restype = ctypes.c_size_t
        lib.w4a16_quantize.argtypes = [_p, _i64, _i64, _p, _p, _p]
        lib.w4a16_gemv.argtypes = [_p, _p, _p, _i64, _i64, _p, _p]
        lib.w4a16_gemm.argtypes = [_p, _i64, _p, _p, _i64, _i64, _p, _p]
        lib.w4a16_gemm_ex.argtypes = [_p, _i64, _p, _p, _i64, _i64, _p, ctypes.c_int, _p]
        lib.w4a16_gemm_workspace_bytes.argtypes = [_i64, _i64, _i64]
        lib.w4a16_gemm_workspace_bytes.restype = ctypes.c_size_t
        lib.w4a16_gemm_ws.argtypes = [_p, _i64, _p, _p, _i64, _i64, _p, _p, ctypes.c_size_t, _p]
        lib.w4a16_gemm_ws.restype = ctypes.c_int
        lib.w4a16_gemm_asym_workspace_bytes.argtypes = [_i64, _i64, _i64, _i64]
        lib.w4a16_gemm_asym_workspace_bytes.restype = ctypes.c_size_t
        lib.w4a16_gemm_asym_ws.argtypes = [_p, _i64, _p, _p, _p, _i64, _i64, _i64, _p, _p,
                                           ctypes.c_size_t, _p]
        lib.w4a16_gemm_asym_ws.restype = ctypes.c_int
        lib.w4a16_scales_bytes_g.argtypes = [_i64, _i64, _i64]
        lib.w4a16_scales_bytes_g.restype = ctypes.c_size_t
        lib.w4a16_quantize_g.argtypes = [_p, _i64, _i64, _i64, _p, _p, _p]
        lib.w4a16_gemv_g.argtypes = [_p, _p, _p, _i64, _i64, _i64, _p, _p]
        lib.w4a16_gemm_g.argtypes = [_p, _i64, _p, _p, _i64, _i64, _i64, _p, _p]
        lib.w4a16_quantize_perm.argtypes = [_p, _p, _i64, _i64, _p, _p, _p]
        lib.w4a16_gemv_perm.argtypes = [_p, _p, _p, _p, _i64, _i64, _p, _p]
        lib.w4a16_gemm_perm.argtypes = [_p, _i64, _p, _p, _p, _i64, _i64, _p, _p]
        lib.w4a16_quantize_asym.argtypes = [_p, _p, _i64, _i64, _i64, _p, _p, _p, _p]
        lib.w4a16_gemv_asym.argtypes = [_p, _p, _p, _p, _p, _i64, _i64, _i64, _p, _p]
        lib.w4a16_gemm_asym.argtypes = [_p, _i64, _p, _p, _p, _p, _i64, _i64, _i64, _p, _p]
        lib.w4a16_linear_workspace_bytes.argtypes = [_i64, _i64, ctypes.c_int]
        lib.w4a16_linear_workspace_bytes.restype = ctypes.c_size_t
        lib.w4a16_linear.argtypes = [_p, _i64, _p, _p, _p, _p, _i64, _i64, _i64, _p, ctypes.c_int,
                                     _p, ctypes.c_size_t, _p]
        lib.w4a16_linear.restype = ctypes.c_int
        lib.w4a16_q4_0_bytes.argtypes = [_i64, _i64]
        lib.w4a16_q4_0_bytes.restype = ctypes.c_size_t
        lib.w4a16_quantize_q4_0.argtypes = [_p, _i64, _i64, _p, _p]
        lib.w4a16_gemv_q4_0.argtypes = [_p, _p, _i64, _i64, _p, _p]
        lib.w4a16_gemm_q4_0.argtypes = [_p, _i64, _p, _i64, _i64, _p, _p]
        for f in (lib.w4a16_quantize_q4_0, lib.w4a16_gemv_q4_0, lib.w4a16_gemm_q4_0):
            f.restype = ctypes.c_int
        for f in (lib.w4a16_quantize, lib.w4a16_gemv, lib.w4a16_gemm, lib.w4a16_gemm_ex,
                  lib.w4a16_quantize_g, lib.w4a16_gemv_g, lib.w4a16_gemm_g,
                  lib.w4a16_quantize_perm, lib.w4a16_gemv_perm, lib.w4a16_gemm_perm,
                  lib.w4a16_quantize_asym, lib.w4a16_gemv_asym, lib.w4a16_gemm_asym):
            f.restype = ctypes.c_int
        lib.w4a16_valu_max_m.restype = ctypes.c_int64
        lib.w4a16_gemv_chain.argtypes = [ctypes.POINTER(GemvStage), ctypes.c_int, _p, _p]
        lib.w4a16_gemv_chain.restype = ctypes.c_int
        lib.w4a16_gemv_chain_noalloc.argtypes = [ctypes.POINTER(GemvStage), ctypes.c_int, _p, _p]
        lib.w4a16_gemv_chain_noalloc.restype = ctypes.c_int
        lib.w4a16_status_string.argtypes = [ctypes.c_int]
        lib.w4a16_status_string.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def status_string(status: int) -> str:
    return library().w4a16_status_string(int(status)).decode()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise W4A16Error(fn, status)


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, ndim: int) -> None:
    if not isinstance(t, torch.Tensor):
        raise ValueError("%s must be a torch.Tensor" % name)
    if t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if t.device.type != "cuda":
        raise ValueError("%s must be on the GPU, got %s" % (name, t.device))
    if t.dim() != ndim:
        raise ValueError("%s must have %d dims, got shape %s" % (name, ndim, tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def packed_bytes(N: int, K: int) -> int:
    return library().w4a16_packed_bytes(N, K)


PER_CHANNEL = -1                          # one scale per row (W4A16_PER_CHANNEL)
GROUPS = (32, 64, 128, 256, PER_CHANNEL)   # elements per scale the kernels take


def scales_per_row(K: int, group: int) -> int:
    """Scales (and zero points) per row of a K-wide weight."""
    return (1 if K > 0 else 0) if group == PER_CHANNEL else K // group


def scales_bytes(N: int, K: int, group: int = W4A16_GROUP) -> int:
    return library().w4a16_scales_bytes_g(N, K, group)


def _check_group(group: int, K: int) -> None:
    if group not in GROUPS:
        raise ValueError("group must be one of %s, got %r" % (GROUPS, group))
    if K % W4A16_GROUP or (group != PER_CHANNEL and K % group):
        raise ValueError("K = %d is not a multiple of %d and of the group %d"
                         % (K, W4A16_GROUP, group))


def _perm(perm, K: int):
    """Checks an act-order column order: int32 [K] on the GPU."""
    _need(perm, "perm", torch.int32, 1)
    if perm.shape[0] != K:
        raise ValueError("perm has %d entries, K = %d" % (perm.shape[0], K))
    return perm


def quantize(W: torch.Tensor, packed: torch.Tensor = None, scales: torch.Tensor = None,
             group: int = W4A16_GROUP, perm: torch.Tensor = None):
    """W fp16 [N, K] -> (packed int32 [N, K/8] holding uint32 words, scales fp16
    [N, K/group]); group 32, 64, 128 (default) or 256.  perm (int32 [K], act
    order, group 128 only): quantize the column-permuted W[:, perm]."""
    lib = library()
    _need(W, "W", torch.float16, 2)
    N, K = W.shape
    _check_group(group, K)
    if perm is not None:
        _perm(perm, K)
        if group != W4A16_GROUP:
            raise ValueError("act order takes group %d" % W4A16_GROUP)
    if packed is None:
        packed = torch.empty((N, K // 8), dtype=torch.int32, device=W.device)
    if scales is None:
        scales = torch.empty((N, scales_per_row(K, group)), dtype=torch.float16,
                             device=W.device)
    _need(packed, "packed", torch.int32, 2)
    _need(scales, "scales", torch.float16, 2)
    if tuple(packed.shape) != (N, K // 8) or tuple(scales.shape) != (N, scales_per_row(K, group)):
        raise ValueError("output shapes do not match W")
    if perm is not None:
        st = lib.w4a16_quantize_perm(W.data_ptr(), perm.data_ptr(), N, K, packed.data_ptr(),
                                     scales.data_ptr(), _stream())
    elif group == W4A16_GROUP:
        st = lib.w4a16_quantize(W.data_ptr(), N, K, packed.data_ptr(), scales.data_ptr(),
                                _stream())
    else:
        st = lib.w4a16_quantize_g(W.data_ptr(), N, K, group, packed.data_ptr(),
                                  scales.data_ptr(), _stream())
    _check("w4a16_quantize", st)
    return packed, scales


def _weights(packed: torch.Tensor, scales: torch.Tensor):
    """(N, K, group) of a packed weight; the group follows from the scales'
    shape [N, K/group]."""
    _need(packed, "packed", torch.int32, 2)
    _need(scales, "scales", torch.float16, 2)
    N, K = packed.shape[0], packed.shape[1] * 8
    ng = scales.shape[1]
    group = K // ng if ng > 0 and K % ng == 0 else 0
    if ng == 1 and group not in GROUPS:
        group = PER_CHANNEL                     # one scale per row
    if scales.shape[0] != N or (K > 0 and group not in GROUPS) or (K == 0 and ng != 0):
        raise ValueError("scales shape %s does not match packed %s"
                         % (tuple(scales.shape), tuple(packed.shape)))
    return N, K, (group if K > 0 else W4A16_GROUP)


def gemv(x: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor,
         y: torch.Tensor = None, perm: torch.Tensor = None) -> torch.Tensor:
    """x fp16 [K] -> y fp16 [N] (decode GEMV, M = 1).  perm: act-order column
    order of the weight (int32 [K]); column j meets x[perm[j]]."""
    lib = library()
    N, K, group = _weights(packed, scales)
    _need(x, "x", torch.float16, 1)
    if x.shape[0] != K:
        raise ValueError("x has %d elements, K = %d" % (x.shape[0], K))
    if y is None:
        y = torch.empty((N,), dtype=torch.float16, device=x.device)
    _need(y, "y", torch.float16, 1)
    if y.shape[0] != N:
        raise ValueError("y has %d elements, N = %d" % (y.shape[0], N))
    if perm is not None:
        _perm(perm, K)
        if group != W4A16_GROUP:
            raise ValueError("act order takes group %d" % W4A16_GROUP)
        st = lib.w4a16_gemv_perm(x.data_ptr(), perm.data_ptr(), packed.data_ptr(),
                                 scales.data_ptr(), N, K, y.data_ptr(), _stream())
    elif group == W4A16_GROUP:
        st = lib.w4a16_gemv(x.data_ptr(), packed.data_ptr(), scales.data_ptr(), N, K,
                            y.data_ptr(), _stream())
    else:
        st = lib.w4a16_gemv_g(x.data_ptr(), packed.data_ptr(), scales.data_ptr(), N, K, group,
                              y.data_ptr(), _stream())
    _check("w4a16_gemv", st)
    return y


def gemm(X: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor, algo=None,
         Y: torch.Tensor = None, perm: torch.Tensor = None) -> torch.Tensor:
    """X fp16 [M, K] -> Y fp16 [M, N].  algo: None/'auto', 'valu' or 'mfma'.
    perm: act-order column order (int32 [K]); Y = X[:, perm] . Ŵᵀ."""
    N, K, group = _weights(packed, scales)
    if algo not in _ALGOS:
        raise ValueError("algo must be one of %s" % sorted(k for k in _ALGOS if k))
    if group == W4A16_GROUP and perm is None:
        lib = library()
        X, Y, M = _rows(X, K, N, Y)
        st = lib.w4a16_gemm_ex(X.data_ptr(), M, packed.data_ptr(), scales.data_ptr(), N, K,
                               Y.data_ptr(), _ALGOS[algo], _stream())
        _check("w4a16_gemm", st)
        return Y
    if algo in (None, "auto"):
        lib = library()
        X, Y, M = _rows(X, K, N, Y)
        if perm is not None:
            _perm(perm, K)
            if group != W4A16_GROUP:
                return linear(X, packed, scales, perm=perm, Y=Y)
            st = lib.w4a16_gemm_perm(X.data_ptr(), M, perm.data_ptr(), packed.data_ptr(),
                                     scales.data_ptr(), N, K, Y.data_ptr(), _stream())
        else:
            st = lib.w4a16_gemm_g(X.data_ptr(), M, packed.data_ptr(), scales.data_ptr(), N, K,
                                  group, Y.data_ptr(), _stream())
        _check("w4a16_gemm", st)
        return Y
    return linear(X, packed, scales, perm=perm, algo=algo, Y=Y)


def _rows(X: torch.Tensor, K: int, N: int, Y: torch.Tensor):
    _need(X, "X", torch.float16, 2)
    M = X.shape[0]
    if X.shape[1] != K:
        raise ValueError("X has %d columns, K = %d" % (X.shape[1], K))
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.float16, device=X.device)
    _need(Y, "Y", torch.float16, 2)
    if tuple(Y.shape) != (M, N):
        raise ValueError("Y shape %s, want %s" % (tuple(Y.shape), (M, N)))
    return X, Y, M


def linear_workspace(M: int, K: int, device="cuda") -> torch.Tensor:
    """Workspace for linear() with a perm (the act-order copy of X): uint8
    of w4a16_linear_workspace_bytes(M, K, 1) bytes."""
    n = library().w4a16_linear_workspace_bytes(M, K, 1)
    return torch.empty(max(int(n), 1), dtype=torch.uint8, device=device)


def linear(X: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor,
           zeros: torch.Tensor = None, perm: torch.Tensor = None, algo=None,
           Y: torch.Tensor = None, workspace: torch.Tensor = None) -> torch.Tensor:
    """The linear layer with every option (w4a16_linear): group from the
    scales' shape, asymmetric weights when zeros is given, act order when
    perm is given; algo None/'auto', 'valu' or 'mfma'; workspace from
    linear_workspace() (optional)."""
    lib = library()
    N, K, group = _weights(packed, scales)
    if algo not in _ALGOS:
        raise ValueError("algo must be one of %s" % sorted(k for k in _ALGOS if k))
    if zeros is not None:
        _zeros(zeros, scales)
    if perm is not None:
        _perm(perm, K)
    X, Y, M = _rows(X, K, N, Y)
    ws, ws_bytes = None, 0
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8, 1)
        ws, ws_bytes = workspace.data_ptr(), workspace.numel()
    st = lib.w4a16_linear(X.data_ptr(), M, perm.data_ptr() if perm is not None else None,
                          packed.data_ptr(), scales.data_ptr(),
                          zeros.data_ptr() if zeros is not None else None, N, K, group,
                          Y.data_ptr(), _ALGOS[algo], ws, ws_bytes, _stream())
    _check("w4a16_linear", st)
    return Y


def gemm_workspace(M: int, N: int, K: int, device="cuda") -> torch.Tensor:
    """A zeroed workspace for gemm_ws (uint8, at least 1 byte; the library
    keeps it reusable across calls)."""
    n = library().w4a16_gemm_workspace_bytes(M, N, K)
    return torch.zeros(max(1, n), dtype=torch.uint8, device=device)


def gemm_ws(X: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor,
            workspace: torch.Tensor, Y: torch.Tensor = None) -> torch.Tensor:
    """w4a16_gemm_ws: gemm (automatic kernel choice, group 128) with K split
    over blocks through `workspace` (from gemm_workspace) where the library
    splits the shape."""
    lib = library()
    N, K, group = _weights(packed, scales)
    if group != W4A16_GROUP:
        raise ValueError("gemm_ws takes group %d weights" % W4A16_GROUP)
    _need(X, "X", torch.float16, 2)
    M = X.shape[0]
    if X.shape[1] != K:
        raise ValueError("X has %d columns, K = %d" % (X.shape[1], K))
    _need(workspace, "workspace", torch.uint8, 1)
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.float16, device=X.device)
    _need(Y, "Y", torch.float16, 2)
    if tuple(Y.shape) != (M, N):
        raise ValueError("Y shape %s, want %s" % (tuple(Y.shape), (M, N)))
    _check("w4a16_gemm_ws", lib.w4a16_gemm_ws(X.data_ptr(), M, packed.data_ptr(),
                                              scales.data_ptr(), N, K, Y.data_ptr(),
                                              workspace.data_ptr(), workspace.numel(),
                                              _stream()))
    return Y


def quantize_asym(W: torch.Tensor, packed: torch.Tensor = None, scales: torch.Tensor = None,
                  zeros: torch.Tensor = None, group: int = W4A16_GROUP,
                  perm: torch.Tensor = None):
    """Asymmetric INT4: W fp16 [N, K] -> (packed int32 [N, K/8] with nibbles
    q in [0, 15], scales fp16 [N, K/group], zeros int16 [N, K/group]);
    ŵ = s * (q - z).  perm (int32 [K]): quantize W[:, perm] (act order)."""
    lib = library()
    _need(W, "W", torch.float16, 2)
    N, K = W.shape
    _check_group(group, K)
    if perm is not None:
        _perm(perm, K)
    if packed is None:
        packed = torch.empty((N, K // 8), dtype=torch.int32, device=W.device)
    if scales is None:
        scales = torch.empty((N, scales_per_row(K, group)), dtype=torch.float16,
                             device=W.device)
    if zeros is None:
        zeros = torch.empty((N, scales_per_row(K, group)), dtype=torch.int16, device=W.device)
    _need(packed, "packed", torch.int32, 2)
    _need(scales, "scales", torch.float16, 2)
    _need(zeros, "zeros", torch.int16, 2)
    ng = scales_per_row(K, group)
    if (tuple(packed.shape) != (N, K // 8) or tuple(scales.shape) != (N, ng)
            or tuple(zeros.shape) != (N, ng)):
        raise ValueError("output shapes do not match W")
    st = lib.w4a16_quantize_asym(W.data_ptr(), perm.data_ptr() if perm is not None else None,
                                 N, K, group, packed.data_ptr(), scales.data_ptr(),
                                 zeros.data_ptr(), _stream())
    _check("w4a16_quantize_asym", st)
    return packed, scales, zeros


def _zeros(zeros: torch.Tensor, scales: torch.Tensor) -> None:
    _need(zeros, "zeros", torch.int16, 2)
    if zeros.shape != scales.shape:
        raise ValueError("zeros shape %s, scales %s" % (tuple(zeros.shape), tuple(scales.shape)))


def gemv_asym(x: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor,
              zeros: torch.Tensor, y: torch.Tensor = None,
              perm: torch.Tensor = None) -> torch.Tensor:
    """Asymmetric weights: x fp16 [K] -> y fp16 [N] (M = 1)."""
    lib = library()
    N, K, group = _weights(packed, scales)
    _zeros(zeros, scales)
    _need(x, "x", torch.float16, 1)
    if x.shape[0] != K:
        raise ValueError("x has %d elements, K = %d" % (x.shape[0], K))
    if y is None:
        y = torch.empty((N,), dtype=torch.float16, device=x.device)
    _need(y, "y", torch.float16, 1)
    if y.shape[0] != N:
        raise ValueError("y has %d elements, N = %d" % (y.shape[0], N))
    if perm is not None:
        _perm(perm, K)
    st = lib.w4a16_gemv_asym(x.data_ptr(), perm.data_ptr() if perm is not None else None,
                             packed.data_ptr(), scales.data_ptr(), zeros.data_ptr(), N, K, group,
                             y.data_ptr(), _stream())
    _check("w4a16_gemv_asym", st)
    return y


def gemm_asym(X: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor,
              zeros: torch.Tensor, Y: torch.Tensor = None,
              perm: torch.Tensor = None, algo=None) -> torch.Tensor:
    """Asymmetric weights: X fp16 [M, K] -> Y fp16 [M, N] (VALU path for
    small M, matrix cores above; algo forces one as for gemm)."""
    if algo not in (None, "auto"):
        return linear(X, packed, scales, zeros=zeros, perm=perm, algo=algo, Y=Y)
    lib = library()
    N, K, group = _weights(packed, scales)
    _zeros(zeros, scales)
    X, Y, M = _rows(X, K, N, Y)
    if perm is not None:
        _perm(perm, K)
    st = lib.w4a16_gemm_asym(X.data_ptr(), M, perm.data_ptr() if perm is not None else None,
                             packed.data_ptr(), scales.data_ptr(), zeros.data_ptr(), N, K, group,
                             Y.data_ptr(), _stream())
    _check("w4a16_gemm_asym", st)
    return Y


def gemm_asym_workspace(M: int, N: int, K: int, group: int = W4A16_GROUP,
                        device="cuda") -> torch.Tensor:
    """A workspace for gemm_asym_ws (uint8, at least 1 byte)."""
    n = library().w4a16_gemm_asym_workspace_bytes(M, N, K, group)
    return torch.empty(max(1, n), dtype=torch.uint8, device=device)


def gemm_asym_ws(X: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor,
                 zeros: torch.Tensor, workspace: torch.Tensor,
                 Y: torch.Tensor = None) -> torch.Tensor:
    """w4a16_gemm_asym_ws: gemm_asym (no perm) with K split over blocks
    through `workspace` (from gemm_asym_workspace) where the library splits
    the shape."""
    lib = library()
    N, K, group = _weights(packed, scales)
    _zeros(zeros, scales)
    X, Y, M = _rows(X, K, N, Y)
    _need(workspace, "workspace", torch.uint8, 1)
    _check("w4a16_gemm_asym_ws",
           lib.w4a16_gemm_asym_ws(X.data_ptr(), M, packed.data_ptr(), scales.data_ptr(),
                                  zeros.data_ptr(), N, K, group, Y.data_ptr(),
                                  workspace.data_ptr(), workspace.numel(), _stream()))
    return Y


Q4_0_BLOCK_BYTES = 18      # fp16 d + 16 code bytes per 32 elements


def q4_0_blocks(N: int, K: int, device="cuda") -> torch.Tensor:
    """An uninitialised Q4_0 buffer: a uint8 [N, K/32 * 18] view of storage
    rounded up to 16 bytes (the padding the library's 16-byte loads read)."""
    nbytes = N * (K // 32) * Q4_0_BLOCK_BYTES
    flat = torch.empty(((nbytes + 15) // 16 * 16,), dtype=torch.uint8, device=device)
    return flat[:nbytes].view(N, K // 32 * Q4_0_BLOCK_BYTES)


def _q4_0_storage(blocks: torch.Tensor) -> None:
    need = (blocks.numel() + 15) // 16 * 16
    have = blocks.untyped_storage().nbytes() - blocks.storage_offset()
    if have < need:
        raise ValueError("the Q4_0 buffer needs %d bytes of storage (blocks rounded up to 16), "
                         "has %d; allocate it with q4_0_blocks()" % (need, have))


def quantize_q4_0(W: torch.Tensor, blocks: torch.Tensor = None) -> torch.Tensor:
    """W fp16 [N, K] -> Q4_0 blocks, uint8 [N, K/32 * 18] (see q4_0_blocks)."""
    lib = library()
    _need(W, "W", torch.float16, 2)
    N, K = W.shape
    if K % W4A16_GROUP:
        raise ValueError("K = %d is not a multiple of %d" % (K, W4A16_GROUP))
    if blocks is None:
        blocks = q4_0_blocks(N, K, device=W.device)
    _need(blocks, "blocks", torch.uint8, 2)
    if tuple(blocks.shape) != (N, K // 32 * Q4_0_BLOCK_BYTES):
        raise ValueError("blocks shape %s, want %s"
                         % (tuple(blocks.shape), (N, K // 32 * Q4_0_BLOCK_BYTES)))
    _q4_0_storage(blocks)
    _check("w4a16_quantize_q4_0",
           lib.w4a16_quantize_q4_0(W.data_ptr(), N, K, blocks.data_ptr(), _stream()))
    return blocks


def _q4_0_shape(blocks: torch.Tensor):
    _need(blocks, "blocks", torch.uint8, 2)
    N, nbytes = blocks.shape
    if nbytes % Q4_0_BLOCK_BYTES:
        raise ValueError("blocks rows of %d bytes are not whole 18-byte blocks" % nbytes)
    _q4_0_storage(blocks)
    return N, nbytes // Q4_0_BLOCK_BYTES * 32


def gemv_q4_0(x: torch.Tensor, blocks: torch.Tensor, y: torch.Tensor = None) -> torch.Tensor:
    """Q4_0 weights: x fp16 [K] -> y fp16 [N]."""
    lib = library()
    N, K = _q4_0_shape(blocks)
    _need(x, "x", torch.float16, 1)
    if x.shape[0] != K:
        raise ValueError("x has %d elements, K = %d" % (x.shape[0], K))
    if y is None:
        y = torch.empty((N,), dtype=torch.float16, device=x.device)
    _need(y, "y", torch.float16, 1)
    if y.shape[0] != N:
        raise ValueError("y has %d elements, N = %d" % (y.shape[0], N))
    _check("w4a16_gemv_q4_0", lib.w4a16_gemv_q4_0(x.data_ptr(), blocks.data_ptr(), N, K,
                                                  y.data_ptr(), _stream()))
    return y


def gemm_q4_0(X: torch.Tensor, blocks: torch.Tensor, Y: torch.Tensor = None) -> torch.Tensor:
    """Q4_0 weights: X fp16 [M, K] -> Y fp16 [M, N]."""
    lib = library()
    N, K = _q4_0_shape(blocks)
    _need(X, "X", torch.float16, 2)
    M = X.shape[0]
    if X.shape[1] != K:
        raise ValueError("X has %d columns, K = %d" % (X.shape[1], K))
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.float16, device=X.device)
    _need(Y, "Y", torch.float16, 2)
    if tuple(Y.shape) != (M, N):
        raise ValueError("Y shape %s, want %s" % (tuple(Y.shape), (M, N)))
    _check("w4a16_gemm_q4_0", lib.w4a16_gemm_q4_0(X.data_ptr(), M, blocks.data_ptr(), N, K,
                                                  Y.data_ptr(), _stream()))
    return Y


def chain_sync_buffer(device="cuda") -> torch.Tensor:
    """A zeroed sync buffer for gemv_chain (W4A16_CHAIN_SYNC_WORDS int32)."""
    return torch.zeros(CHAIN_SYNC_WORDS, dtype=torch.int32, device=device)


class W4A16ChainError(RuntimeError):
    """A wait between the stages of a gemv_chain launch gave up: the grid was
    not co-resident (the GPU was shared), so outputs may be stale."""


def chain_error(sync: torch.Tensor) -> bool:
    """True when the sticky error word of a gemv_chain sync buffer is set
    (reads the word: synchronizes with the current stream)."""
    return int(sync[CHAIN_ERR_WORD].item()) != 0


def _chain_stages(stages):
    arr = (GemvStage * max(1, len(stages)))()
    for i, (x, packed, scales, y) in enumerate(stages):
        N, K, group = _weights(packed, scales)
        if group != W4A16_GROUP:
            raise ValueError("stage %d: gemv_chain takes group %d weights" % (i, W4A16_GROUP))
        _need(x, "x", torch.float16, 1)
        _need(y, "y", torch.float16, 1)
        if x.shape[0] != K or y.shape[0] != N:
            raise ValueError("stage %d: x has %d elements (K = %d), y %d (N = %d)"
                             % (i, x.shape[0], K, y.shape[0], N))
        arr[i] = GemvStage(x.data_ptr(), packed.data_ptr(), scales.data_ptr(), y.data_ptr(),
                           N, K)
    return arr


def gemv_chain_noalloc(stages, status: torch.Tensor) -> None:
    """w4a16_gemv_chain_noalloc: gemv_chain with the library's own counters
    (no sync buffer).  status: int32 [1] device tensor; after the launch it
    holds 0, or non-zero when a wait between stages gave up (the caller reads
    it when convenient)."""
    lib = library()
    if len(stages) > CHAIN_MAX:
        raise ValueError("at most %d stages per call" % CHAIN_MAX)
    _need(status, "status", torch.int32, 1)
    if status.shape[0] < 1:
        raise ValueError("status needs one element")
    arr = _chain_stages(stages)
    _check("w4a16_gemv_chain_noalloc",
           lib.w4a16_gemv_chain_noalloc(arr, len(stages), status.data_ptr(), _stream()))


def gemv_chain(stages, sync: torch.Tensor, check: bool = True) -> None:
    """Run a dependent sequence of decode GEMVs in one launch.

    stages: list of (x [K], packed [N, K/8], scales [N, K/128], y [N]) device
    tensors; x of a stage may be the y of an earlier stage (or a view of it).
    sync: int32 [CHAIN_SYNC_WORDS] device tensor from chain_sync_buffer().
    check: after the launch, read the sync buffer's error word (this waits
    for the launch) and raise W4A16ChainError if a wait between stages gave
    up.  Skipped while the current stream is being captured into a graph;
    callers that replay a graph (or pass check=False) test chain_error(sync)
    themselves.
    """
    lib = library()
    if len(stages) > CHAIN_MAX:
        raise ValueError("at most %d stages per call" % CHAIN_MAX)
    _need(sync, "sync", torch.int32, 1)
    if sync.shape[0] < CHAIN_SYNC_WORDS:
        raise ValueError("sync needs %d words" % CHAIN_SYNC_WORDS)
    arr = _chain_stages(stages)
    _check("w4a16_gemv_chain", lib.w4a16_gemv_chain(arr, len(stages), sync.data_ptr(),
                                                    _stream()))
    if check and not torch.cuda.is_current_stream_capturing() and chain_error(sync):
        raise W4A16ChainError("w4a16_gemv_chain: a wait between stages gave up (error word "
                              "set); the outputs may be stale")


def valu_max_m() -> int:
    return library().w4a16_valu_max_m()

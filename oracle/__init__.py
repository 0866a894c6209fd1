"""CPU oracle of the W4A16 linear layer — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the HIP library
in ``weight_only_int4_gemv_amd`` and never imports it.

The arithmetic lives in ``w4a16_oracle.c`` (plain C, binary64), written from
the quantization equations of the qaqbuyan.com quantization article
(section "量化的数学基石——从 IEEE 754 到量化误差", sub-sections 1-3) and
the INT4 paragraph of the guijiagi.com "量化" tag page.  This module only
compiles it with gcc, loads it with ctypes and marshals numpy arrays.

Every function here is pinned by ``tests/test_oracle_pins.py``; nothing is
"parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "w4a16_oracle.c")
LIBRARY = os.path.join(_HERE, "liboracle_w4a16.so")
CFLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC",
          "-std=c11", "-Wall", "-Wextra"]

_i64 = ctypes.c_int64
_p = ctypes.c_void_p


def compile_library(source: str = SOURCE, output: str = LIBRARY) -> str:
    """Compile the oracle C source to a shared library with gcc."""
    tmp = output + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", *CFLAGS, "-o", tmp, source, "-lm"], check=True)
    os.replace(tmp, output)
    return output


class Oracle:
    """ctypes front end of one compiled oracle library (numpy in, numpy out)."""

    def __init__(self, library: str = LIBRARY):
        lib = ctypes.CDLL(library)
        lib.oracle_f64_from_f16.argtypes = [ctypes.c_uint16]
        lib.oracle_f64_from_f16.restype = ctypes.c_double
        lib.oracle_f16_from_f64.argtypes = [ctypes.c_double]
        lib.oracle_f16_from_f64.restype = ctypes.c_uint16
        lib.oracle_quantize.argtypes = [_p, _i64, _i64, _i64, _p, _p]
        lib.oracle_dequantize.argtypes = [_p, _p, _i64, _i64, _i64, _p]
        lib.oracle_matmul.argtypes = [_p, _i64, _p, _p, _i64, _i64, _i64, _p, _p]
        lib.oracle_matmul_sampled.argtypes = [_p, _i64, _p, _p, _i64, _i64, _i64, _p, _p, _i64,
                                              _p, _p]
        lib.oracle_quantize_asym.argtypes = [_p, _i64, _i64, _i64, _p, _p, _p]
        lib.oracle_dequantize_asym.argtypes = [_p, _p, _p, _i64, _i64, _i64, _p]
        lib.oracle_matmul_asym.argtypes = [_p, _i64, _p, _p, _p, _i64, _i64, _i64, _p, _p]
        lib.oracle_quantize_q4_0.argtypes = [_p, _i64, _i64, _p]
        lib.oracle_dequantize_q4_0.argtypes = [_p, _i64, _i64, _p]
        lib.oracle_matmul_q4_0.argtypes = [_p, _i64, _p, _i64, _i64, _p, _p]
        for f in (lib.oracle_quantize, lib.oracle_dequantize, lib.oracle_matmul,
                  lib.oracle_matmul_sampled, lib.oracle_quantize_asym,
                  lib.oracle_dequantize_asym, lib.oracle_matmul_asym,
                  lib.oracle_quantize_q4_0, lib.oracle_dequantize_q4_0,
                  lib.oracle_matmul_q4_0):
            f.restype = ctypes.c_int
        lib.oracle_num_threads.restype = ctypes.c_int
        self.lib = lib
        self.path = library

    # -- fp16 codec ---------------------------------------------------------
    def f64_from_f16(self, bits: int) -> float:
        return self.lib.oracle_f64_from_f16(int(bits))

    def f16_from_f64(self, value: float) -> int:
        return self.lib.oracle_f16_from_f64(float(value))

    # -- quantizer ----------------------------------------------------------
    def quantize(self, W: np.ndarray, group: int = 128):
        """W: fp16 [N, K] (float16 or its uint16 bits) -> (packed uint32 [N, K/8],
        scales uint16 bits [N, K/group])."""
        W = _bits16(W)
        N, K = W.shape
        packed = np.zeros((N, K // 8), dtype=np.uint32)
        scales = np.zeros((N, K // group), dtype=np.uint16)
        rc = self.lib.oracle_quantize(_ptr(W), N, K, group, _ptr(packed), _ptr(scales))
        if rc != 0:
            raise ValueError("oracle_quantize: bad sizes N=%d K=%d group=%d" % (N, K, group))
        return packed, scales

    def dequantize(self, packed: np.ndarray, scales: np.ndarray, group: int = 128) -> np.ndarray:
        """Exact Ŵ = s*q as float64 [N, K]."""
        packed = np.ascontiguousarray(packed, dtype=np.uint32)
        scales = _bits16(scales)
        N, K = packed.shape[0], packed.shape[1] * 8
        out = np.empty((N, K), dtype=np.float64)
        rc = self.lib.oracle_dequantize(_ptr(packed), _ptr(scales), N, K, group, _ptr(out))
        if rc != 0:
            raise ValueError("oracle_dequantize: bad sizes")
        return out

    # -- linear layer -------------------------------------------------------
    def matmul(self, X: np.ndarray, packed: np.ndarray, scales: np.ndarray, group: int = 128):
        """X fp16 [M, K] -> (Y float64 [M, N], Yabs float64 [M, N]) with
        Y = X·Ŵᵀ and Yabs = sum_k |X[m,k] Ŵ[n,k]|."""
        X = _bits16(X)
        if X.ndim == 1:
            X = X.reshape(1, -1)
        packed = np.ascontiguousarray(packed, dtype=np.uint32)
        scales = _bits16(scales)
        M, K = X.shape
        N = packed.shape[0]
        if packed.shape[1] * 8 != K:
            raise ValueError("K mismatch")
        Y = np.empty((M, N), dtype=np.float64)
        Yabs = np.empty((M, N), dtype=np.float64)
        rc = self.lib.oracle_matmul(_ptr(X), M, _ptr(packed), _ptr(scales), N, K, group,
                                    _ptr(Y), _ptr(Yabs))
        if rc != 0:
            raise ValueError("oracle_matmul: bad sizes")
        return Y, Yabs

    def matmul_sampled(self, X, packed, scales, rows, cols, group: int = 128):
        """Outputs Y[rows[i], cols[i]] only (for full-size problems)."""
        X = _bits16(X)
        if X.ndim == 1:
            X = X.reshape(1, -1)
        packed = np.ascontiguousarray(packed, dtype=np.uint32)
        scales = _bits16(scales)
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        cols = np.ascontiguousarray(cols, dtype=np.int64)
        M, K = X.shape
        N = packed.shape[0]
        Y = np.empty(rows.shape[0], dtype=np.float64)
        Yabs = np.empty(rows.shape[0], dtype=np.float64)
        rc = self.lib.oracle_matmul_sampled(_ptr(X), M, _ptr(packed), _ptr(scales), N, K, group,
                                            _ptr(rows), _ptr(cols), rows.shape[0],
                                            _ptr(Y), _ptr(Yabs))
        if rc != 0:
            raise ValueError("oracle_matmul_sampled: bad sizes or indices")
        return Y, Yabs

    # -- asymmetric INT4 ---------------------------------------------------
    def quantize_asym(self, W: np.ndarray, group: int = 128):
        """W: fp16 [N, K] -> (packed uint32 [N, K/8] with nibbles q in [0, 15],
        scales uint16 bits [N, K/group], zero points int16 [N, K/group])."""
        W = _bits16(W)
        N, K = W.shape
        packed = np.zeros((N, K // 8), dtype=np.uint32)
        scales = np.zeros((N, K // group), dtype=np.uint16)
        zeros = np.zeros((N, K // group), dtype=np.int16)
        rc = self.lib.oracle_quantize_asym(_ptr(W), N, K, group, _ptr(packed), _ptr(scales),
                                           _ptr(zeros))
        if rc != 0:
            raise ValueError("oracle_quantize_asym: bad sizes N=%d K=%d group=%d" % (N, K, group))
        return packed, scales, zeros

    def dequantize_asym(self, packed, scales, zeros, group: int = 128) -> np.ndarray:
        """Exact Ŵ = s*(q - z) as float64 [N, K]."""
        packed = np.ascontiguousarray(packed, dtype=np.uint32)
        scales = _bits16(scales)
        zeros = np.ascontiguousarray(zeros, dtype=np.int16)
        N, K = packed.shape[0], packed.shape[1] * 8
        out = np.empty((N, K), dtype=np.float64)
        rc = self.lib.oracle_dequantize_asym(_ptr(packed), _ptr(scales), _ptr(zeros), N, K,
                                             group, _ptr(out))
        if rc != 0:
            raise ValueError("oracle_dequantize_asym: bad sizes")
        return out

    def matmul_asym(self, X, packed, scales, zeros, group: int = 128):
        """(Y, Yabs) of X·Ŵᵀ with the asymmetric Ŵ = s*(q - z)."""
        X = _bits16(X)
        if X.ndim == 1:
            X = X.reshape(1, -1)
        packed = np.ascontiguousarray(packed, dtype=np.uint32)
        scales = _bits16(scales)
        zeros = np.ascontiguousarray(zeros, dtype=np.int16)
        M, K = X.shape
        N = packed.shape[0]
        if packed.shape[1] * 8 != K:
            raise ValueError("K mismatch")
        Y = np.empty((M, N), dtype=np.float64)
        Yabs = np.empty((M, N), dtype=np.float64)
        rc = self.lib.oracle_matmul_asym(_ptr(X), M, _ptr(packed), _ptr(scales), _ptr(zeros),
                                         N, K, group, _ptr(Y), _ptr(Yabs))
        if rc != 0:
            raise ValueError("oracle_matmul_asym: bad sizes")
        return Y, Yabs

    # -- Q4_0 blocks -------------------------------------------------------
    def quantize_q4_0(self, W: np.ndarray) -> np.ndarray:
        """W fp16 [N, K] -> Q4_0 blocks, uint8 [N, K/32 * 18]."""
        W = _bits16(W)
        N, K = W.shape
        blocks = np.zeros((N, K // 32 * 18), dtype=np.uint8)
        rc = self.lib.oracle_quantize_q4_0(_ptr(W), N, K, _ptr(blocks))
        if rc != 0:
            raise ValueError("oracle_quantize_q4_0: bad sizes N=%d K=%d" % (N, K))
        return blocks

    def dequantize_q4_0(self, blocks: np.ndarray, K: int) -> np.ndarray:
        blocks = np.ascontiguousarray(blocks, dtype=np.uint8)
        N = blocks.shape[0]
        out = np.empty((N, K), dtype=np.float64)
        rc = self.lib.oracle_dequantize_q4_0(_ptr(blocks), N, K, _ptr(out))
        if rc != 0:
            raise ValueError("oracle_dequantize_q4_0: bad sizes")
        return out

    def matmul_q4_0(self, X: np.ndarray, blocks: np.ndarray):
        X = _bits16(X)
        if X.ndim == 1:
            X = X.reshape(1, -1)
        blocks = np.ascontiguousarray(blocks, dtype=np.uint8)
        M, K = X.shape
        N = blocks.shape[0]
        if blocks.shape[1] != K // 32 * 18:
            raise ValueError("K mismatch")
        Y = np.empty((M, N), dtype=np.float64)
        Yabs = np.empty((M, N), dtype=np.float64)
        rc = self.lib.oracle_matmul_q4_0(_ptr(X), M, _ptr(blocks), N, K, _ptr(Y), _ptr(Yabs))
        if rc != 0:
            raise ValueError("oracle_matmul_q4_0: bad sizes")
        return Y, Yabs

    def num_threads(self) -> int:
        return self.lib.oracle_num_threads()


def _bits16(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype == np.float16:
        return a.view(np.uint16)
    if a.dtype != np.uint16:
        raise TypeError("expected float16 or uint16 bits, got %s" % a.dtype)
    return a


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


_default = None


def get() -> Oracle:
    """The oracle built from ``w4a16_oracle.c`` (compiled on first use if absent
    or older than its source)."""
    global _default
    if _default is None:
        if (not os.path.exists(LIBRARY)
                or os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE)):
            compile_library()
        _default = Oracle(LIBRARY)
    return _default


def tolerance(y_ref: np.ndarray, y_abs: np.ndarray) -> np.ndarray:
    """Allowed |y - y_ref| per output element:
    1e-3 * sum_k |x_k w_k| + max(2^-10 |y_ref|, 2^-24).

    The second term is the allowance for storing y in fp16 (two half-ulps
    of a normal fp16 value).  Below the smallest normal fp16 (2^-14) the
    fp16 grid is uniform with step 2^-24, so there it is one step: even the
    correctly rounded fp16(y_ref) can sit 2^-25 from y_ref, which 2^-10
    |y_ref| alone would not allow."""
    return 1e-3 * np.asarray(y_abs) + np.maximum(2.0 ** -10 * np.abs(np.asarray(y_ref)),
                                                 2.0 ** -24)

"""The C oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only, OpenMP off).

Every parity verdict rests on ``oracle/w4a16_oracle.c``, which indexes raw
int64 offsets and allocates per-row scratch; an out-of-bounds access or an
undefined shift there could still return plausible numbers.  This test
compiles the same source with ``-fsanitize=address,undefined`` (every report
fatal) and runs, in a child interpreter with the sanitizer runtime loaded
first, every oracle pin plus the symmetric, asymmetric, act-order, Q4_0 and
sampled paths on small ragged shapes (one group, several tiles' worth of
rows, K not a power of two).
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

_CHILD = r"""
import sys
import numpy as np
sys.path.insert(0, sys.argv[2])
sys.path.insert(0, sys.argv[3])
import oracle, oracle_pins
from weight_only_int4_gemv_amd import inputs

o = oracle.Oracle(sys.argv[1])
assert o.num_threads() == 1
for pin in oracle_pins.ALL_PINS:
    fails = pin(o)
    assert fails == [], (pin.__name__, fails[:3])
    print("pin", pin.__name__, "ok", flush=True)

# ragged shapes through every entry point of the oracle
for (M, N, K) in [(1, 1, 128), (3, 7, 384), (5, 33, 1152), (2, 130, 256)]:
    W = inputs.weight(N, K, seed=[41, N, K])
    X = inputs.activation(M, K, seed=[42, M, K])
    for g in (32, 64, 128, 256):
        if K % g:
            continue
        p, s = o.quantize(W, group=g)
        Wh = o.dequantize(p, s, group=g)
        Y, Ya = o.matmul(X, p, s, group=g)
        assert np.allclose(Y, X.astype(np.float64) @ Wh.T, rtol=0, atol=1e-9 * (1 + Ya.max()))
        rows = np.array([0, M - 1, M // 2], dtype=np.int64)
        cols = np.array([0, N - 1, N // 2], dtype=np.int64)
        Ys, Yas = o.matmul_sampled(X, p, s, rows, cols, group=g)
        assert np.array_equal(Ys, Y[rows, cols]) and np.array_equal(Yas, Ya[rows, cols])
        pa, sa, za = o.quantize_asym(W, group=g)
        Wa = o.dequantize_asym(pa, sa, za, group=g)
        Ya2, _ = o.matmul_asym(X, pa, sa, za, group=g)
        assert np.allclose(Ya2, X.astype(np.float64) @ Wa.T, rtol=0, atol=1e-6)
    blocks = o.quantize_q4_0(W)
    Wq = o.dequantize_q4_0(blocks, K)
    Yq, _ = o.matmul_q4_0(X, blocks)
    assert np.allclose(Yq, X.astype(np.float64) @ Wq.T, rtol=0, atol=1e-6)
    print("shape", M, N, K, "ok", flush=True)
print("SANITIZED-ORACLE-OK", flush=True)
"""


def _runtime(name):
    out = subprocess.run(["gcc", "-print-file-name=" + name], check=True,
                         capture_output=True, text=True).stdout.strip()
    return out if os.path.isabs(out) and os.path.exists(out) else None


def test_oracle_under_asan_ubsan(tmp_path):
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc has no AddressSanitizer runtime here")
    lib = str(tmp_path / "liboracle_sanitized.so")
    src = os.path.join(ROOT, "oracle", "w4a16_oracle.c")
    # Same language flags as the product oracle build, OpenMP off, every
    # sanitizer report fatal.
    subprocess.run(["gcc", "-O1", "-g", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-fno-fast-math", "-ffp-contract=off", "-std=c11", "-Wall", "-Wextra",
                    "-shared", "-fPIC", "-o", lib, src, "-lm"], check=True)
    env = dict(os.environ)
    # The sanitizer runtime must come first in the process's library list;
    # anything already preloaded stays preloaded after it.
    prior = env.get("LD_PRELOAD", "")
    env["LD_PRELOAD"] = asan + (":" + prior if prior else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["OMP_NUM_THREADS"] = "1"
    proc = subprocess.run([sys.executable, "-c", _CHILD, lib, os.path.join(ROOT, "tests"), ROOT],
                          env=env, capture_output=True, text=True, timeout=600)
    report = proc.stdout[-3000:] + proc.stderr[-6000:]
    assert proc.returncode == 0, report
    assert "SANITIZED-ORACLE-OK" in proc.stdout, report
    assert "runtime error" not in proc.stderr, report
    assert "AddressSanitizer" not in proc.stderr, report

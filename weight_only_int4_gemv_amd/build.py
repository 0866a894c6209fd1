"""Build ``libw4a16.so`` (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

    python -m weight_only_int4_gemv_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(PKG, "libw4a16.so")
SOURCES = ["api.hip", "quantize.hip", "gemv.hip", "gemv_chain.hip", "gemm_mfma.hip",
           "gemm_skinny.hip", "gemv_mfma4.hip", "gemm_batched.hip", "gemv_q4_0.hip",
           "gather_x.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # IEEE fp32 division and no fast-math: the quantizer's integer decisions
    # depend on correctly rounded quotients.
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-fast-math",
    # No packed-fp32 (v_pk_*_f32) instructions anywhere in device code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-I", INCLUDE,
    "-I", CSRC,
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def build(verbose: bool = False) -> str:
    """Compile every source (in parallel) and link the shared library."""
    with tempfile.TemporaryDirectory(prefix="w4a16_build_") as tmp:
        procs = []
        objects = []
        for src in SOURCES:
            obj = os.path.join(tmp, src.replace(".hip", ".o"))
            objects.append(obj)
            cmd = [hipcc(), *HIPCC_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                stderr=subprocess.STDOUT, text=True)))
        failed = []
        for src, p in procs:
            out, _ = p.communicate()
            lines = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln]
            if p.returncode != 0:
                failed.append(src)
                sys.stderr.write("\n".join(lines) + "\n")
            elif verbose and lines:
                print("\n".join(lines))
        if failed:
            raise RuntimeError("hipcc failed on " + ", ".join(failed))
        tmp_lib = LIBRARY + ".tmp%d" % os.getpid()
        cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp_lib, *objects]
        subprocess.run(cmd, check=True, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
        os.replace(tmp_lib, LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

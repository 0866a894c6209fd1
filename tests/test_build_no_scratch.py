"""Every kernel keeps its state in registers and LDS: no scratch memory.

A kernel that falls back to scratch (a lambda left as a call with its
captured arrays in memory, an array indexed at run time) stays correct, so
the parity tests cannot see it, but it runs many times slower.  This test
compiles each HIP source for gfx950 to assembly (no GPU needed) and reads
the kernels' private segment sizes from the code-object metadata.
"""
import os
import re
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

from weight_only_int4_gemv_amd import build as B

# Kernels allowed scratch, with the reason (none).
ALLOWED = set()


def _metadata(src: str, tmp: str):
    out = os.path.join(tmp, os.path.basename(src) + ".s")
    cmd = [B.hipcc(), *B.HIPCC_FLAGS, "--cuda-device-only", "-S", src, "-o", out]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout[-2000:]
    text = open(out).read()
    return [(m.group(1), int(m.group(2))) for m in re.finditer(
        r"\.name:\s+(\S+)\s*\n(?:.*\n)*?\s*\.private_segment_fixed_size:\s+(\d+)", text)]


@pytest.mark.skipif(not os.path.exists(B.hipcc()) and B.hipcc() != "hipcc",
                    reason="hipcc not found")
def test_no_kernel_uses_scratch():
    sources = [os.path.join(B.CSRC, s) for s in B.SOURCES]
    with tempfile.TemporaryDirectory(prefix="w4a16_scratch_") as tmp:
        with ThreadPoolExecutor(max_workers=4) as ex:
            results = list(ex.map(lambda s: _metadata(s, tmp), sources))
    kernels = [k for r in results for k in r]
    assert len(kernels) > 50, "kernel metadata not found"
    bad = [(name, size) for name, size in kernels
           if size > 0 and not any(re.search(a, name) for a in ALLOWED)]
    assert not bad, "kernels using scratch: %s" % bad

"""Checks on the gfx950 assembly of every HIP source (no GPU needed).

1. Every kernel keeps its state in registers and LDS: no scratch memory.
   A kernel that falls back to scratch (a lambda left as a call with its
   captured arrays in memory, an array indexed at run time) stays correct,
   so the parity tests cannot see it, but it runs many times slower.  Read
   from the kernels' private segment sizes in the code-object metadata.

2. No result of a matrix-core instruction is read by a vector instruction
   (ALU, LDS or memory store) before the wait states the matrix core needs,
   on any path through the code.  The hardware does not interlock these
   reads; the compiler inserts s_nop padding, and it has been seen to miss a
   path: an MFMA followed by a branch over another MFMA, with the first
   MFMA's result read right after the join, left 3 wait states on the path
   that skips the branch (the read then returns the register's old value).
   The required counts are the ones the compiler itself pads to inside a
   basic block for the same instructions: 8 after v_mfma_f32_16x16x32_f16,
   5 after v_mfma_f32_4x4x4_16b_f16; each issued instruction counts 1 and
   s_nop N counts N + 1.
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

# wait states before a vector instruction may read an MFMA's destination
MFMA_WAIT_STATES = {"v_mfma_f32_16x16x32_f16": 8, "v_mfma_f32_4x4x4_16b_f16": 5}

pytestmark = pytest.mark.skipif(not os.path.exists(B.hipcc()) and B.hipcc() != "hipcc",
                                reason="hipcc not found")


def _assemble(src: str, tmp: str) -> str:
    out = os.path.join(tmp, os.path.basename(src) + ".s")
    cmd = [B.hipcc(), *B.HIPCC_FLAGS, "--cuda-device-only", "-S", src, "-o", out]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout[-2000:]
    return open(out).read()


@pytest.fixture(scope="module")
def assembly():
    sources = [os.path.join(B.CSRC, s) for s in B.SOURCES]
    with tempfile.TemporaryDirectory(prefix="w4a16_asm_") as tmp:
        with ThreadPoolExecutor(max_workers=4) as ex:
            return dict(zip(B.SOURCES, ex.map(lambda s: _assemble(s, tmp), sources)))


def test_no_kernel_uses_scratch(assembly):
    kernels = []
    for text in assembly.values():
        kernels += [(m.group(1), int(m.group(2))) for m in re.finditer(
            r"\.name:\s+(\S+)\s*\n(?:.*\n)*?\s*\.private_segment_fixed_size:\s+(\d+)", text)]
    assert len(kernels) > 50, "kernel metadata not found"
    bad = [(name, size) for name, size in kernels
           if size > 0 and not any(re.search(a, name) for a in ALLOWED)]
    assert not bad, "kernels using scratch: %s" % bad


# ------------------------------------------------------------ MFMA hazards

def _regs(tok: str):
    m = re.fullmatch(r"([va])\[(\d+):(\d+)\]", tok)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.fullmatch(r"([va])(\d+)", tok)
    return {(m.group(1), int(m.group(2)))} if m else set()


def _split(ins: str):
    parts = ins.split(None, 1)
    ops = [t.strip().split()[0] for t in parts[1].split(",") if t.strip()] if len(parts) > 1 else []
    return parts[0], ops


def _function_body(body: str):
    """Instructions (comments and directives dropped) and label positions."""
    ins, labels = [], {}
    for line in body.split("\n"):
        s = line.split(";")[0].strip()
        if not s:
            continue
        m = re.match(r"^(\.LBB\w+):", s)
        if m:
            labels[m.group(1)] = len(ins)
        elif not s.startswith(".") and not s.endswith(":"):
            ins.append(s)
    return ins, labels


def _successors(i, ins, labels):
    op, ops = _split(ins[i])
    if op == "s_endpgm":
        return []
    if op == "s_branch":
        return [labels[ops[0]]]
    if op.startswith("s_cbranch"):
        return [i + 1, labels[ops[-1]]]
    return [i + 1]


def _reads(op, ops):
    """VGPRs a non-MFMA vector instruction reads."""
    if op.startswith(("ds_write", "ds_store", "buffer_store", "global_store", "flat_store")):
        src = ops
    elif op.startswith("v_") and not op.startswith("v_mfma"):
        src = ops if ("fmac" in op or "_mac_" in op) else ops[1:]
    else:
        return set()
    out = set()
    for t in src:
        out |= _regs(t)
    return out


def mfma_hazards(body: str):
    """(mfma, reader, wait states) for every path on which a vector
    instruction reads an MFMA destination too early; also the MFMA count."""
    ins, labels = _function_body(body)
    found, count = [], 0
    for i, s in enumerate(ins):
        op, ops = _split(s)
        if not op.startswith("v_mfma"):
            continue
        count += 1
        assert op in MFMA_WAIT_STATES, "no wait-state count for %s" % op
        need, dst = MFMA_WAIT_STATES[op], _regs(ops[0])
        stack, best = [(j, 0) for j in _successors(i, ins, labels)], {}
        while stack:
            j, w = stack.pop()
            if j >= len(ins) or w >= need or best.get(j, need) <= w:
                continue
            best[j] = w
            op2, ops2 = _split(ins[j])
            if _reads(op2, ops2) & dst:
                found.append((s, ins[j], w))
                continue
            if op2.startswith("v_") and not op2.startswith(("v_cmp", "v_mfma")) and ops2 \
                    and dst <= _regs(ops2[0]):
                continue                   # destination overwritten: no stale read after
            step = int(ops2[0], 0) + 1 if op2 == "s_nop" else 1
            for k in _successors(j, ins, labels):
                stack.append((k, w + step))
    return found, count


def test_mfma_checker_finds_a_skipped_branch_hazard():
    """The checker itself: a read 3 instructions after the MFMA on the path
    that skips a branch is reported, the padded path is not."""
    body = """
	v_mfma_f32_16x16x32_f16 v[46:49], v[50:53], v[90:93], v[46:49]
	s_cbranch_vccnz .LBB0_2
	v_mfma_f32_16x16x32_f16 v[42:45], v[50:53], v[22:25], v[42:45]
	s_nop 7
.LBB0_2:
	s_andn2_b64 vcc, exec, s[58:59]
	v_fmac_f32_e32 v80, v87, v46
	s_endpgm
"""
    found, count = mfma_hazards(body)
    assert count == 2
    assert len(found) == 1 and "v46" in found[0][1] and found[0][2] == 2


def test_no_mfma_result_read_too_early(assembly):
    total, bad = 0, []
    for src, text in assembly.items():
        for m in re.finditer(r"^(_Z\w+):", text, re.M):
            end = text.find(".Lfunc_end", m.end())
            found, count = mfma_hazards(text[m.end():end])
            total += count
            bad += [(src, m.group(1)[:60]) + f for f in found[:2]]
    assert total > 1000, "MFMA instructions not found"
    assert not bad, "MFMA results read before their wait states: %s" % bad[:6]

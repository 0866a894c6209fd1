"""Plant a mistake in a copy of the oracle (on the CPU) and check that the
pins catch it: every mutant must fail at least one pin."""
import os
import shutil
import subprocess

import pytest

import oracle
import oracle_pins

# (name, text in w4a16_oracle.c, replacement)
MUTANTS = [
    ("round half away from zero", "double r = nearbyint(oracle_f64_from_f16(w[i]) / s);",
     "double r = round(oracle_f64_from_f16(w[i]) / s);"),
    ("round toward zero", "double r = nearbyint(oracle_f64_from_f16(w[i]) / s);",
     "double r = trunc(oracle_f64_from_f16(w[i]) / s);"),
    ("divide by 8 (2^(b-1))", "oracle_f16_from_f64(a / 7.0)", "oracle_f16_from_f64(a / 8.0)"),
    ("q against the unrounded scale", "double r = nearbyint(oracle_f64_from_f16(w[i]) / s);",
     "double r = nearbyint(oracle_f64_from_f16(w[i]) / (a / 7.0));"),
    ("clamp to [-7, 7]", "if (r < -8.0) r = -8.0;", "if (r < -7.0) r = -7.0;"),
    ("no clamp at 7", "if (r > 7.0) r = 7.0;", "if (r > 8.0) r = 8.0;"),
    ("nibble order reversed", "word |= nib << (4 * i);", "word |= nib << (4 * (7 - i));"),
    ("offset 7 instead of 8", "(uint32_t)(q[8 * j + i] + 8) & 0xFu", "(uint32_t)(q[8 * j + i] + 7) & 0xFu"),
    ("unpack offset dropped", "& 0xFu) - 8;", "& 0xFu) - 7;"),
    ("absmax without abs", "double v = fabs(oracle_f64_from_f16(w[i]));",
     "double v = oracle_f64_from_f16(w[i]);"),
    ("fp16 encode truncates", "double r = nearbyint(ldexp(fr, 11));",
     "double r = floor(ldexp(fr, 11));"),
    ("fp16 subnormal decode off by one exponent", "v = ldexp((double)m, -24);",
     "v = ldexp((double)m, -23);"),
    ("scale index uses the wrong group", "oracle_f64_from_f16(row_scales[k / group])",
     "oracle_f64_from_f16(row_scales[(k / group + 1) % (K / group)])"),
    ("matmul drops the first term", "for (int64_t k = 0; k < K; k++) {\n        double w =",
     "for (int64_t k = 1; k < K; k++) {\n        double w ="),
    ("matmul wrong sign", "acc += t;", "acc -= t;"),
    ("activation index transposed", "dot_row(X + m * K, packed + n * (K / 8)",
     "dot_row(X + (M - 1 - m) * K, packed + n * (K / 8)"),
    ("asym: zero point sign flipped", "double z = -nearbyint(mn / s);",
     "double z = nearbyint(mn / s);"),
    ("asym: zero point by floor", "double z = -nearbyint(mn / s);",
     "double z = -floor(mn / s);"),
    ("asym: range over 16 levels", "oracle_f16_from_f64((mx - mn) / 15.0)",
     "oracle_f16_from_f64((mx - mn) / 16.0)"),
    ("asym: range from absmax", "oracle_f16_from_f64((mx - mn) / 15.0)",
     "oracle_f16_from_f64((mx > -mn ? mx : -mn) / 15.0)"),
    ("asym: zero added before rounding", "double r = nearbyint(oracle_f64_from_f16(w[i]) / s) + z;",
     "double r = nearbyint(oracle_f64_from_f16(w[i]) / s + z + 0.5);"),
    ("asym: clamp at 14", "if (r > 15.0) r = 15.0;", "if (r > 14.0) r = 14.0;"),
    ("asym: offset-binary nibble", "word |= ((uint32_t)q[8 * j + i] & 0xFu) << (4 * i);",
     "word |= ((uint32_t)(q[8 * j + i] + 8) & 0xFu) << (4 * i);"),
    ("asym: dequantize ignores z",
     "What[n * K + k] = oracle_f64_from_f16(scales[n * ng + k / group]) *\n"
     "                              (double)(nibble_at(packed + n * (K / 8), k) -\n"
     "                                       zeros[n * ng + k / group]);",
     "What[n * K + k] = oracle_f64_from_f16(scales[n * ng + k / group]) *\n"
     "                              (double)(nibble_at(packed + n * (K / 8), k));"),
    ("q4_0: nibbles of a byte swapped",
     "blk[2 + i] = (uint8_t)(((q[2 * i] + 8) & 0xF) | (((q[2 * i + 1] + 8) & 0xF) << 4));",
     "blk[2 + i] = (uint8_t)(((q[2 * i + 1] + 8) & 0xF) | (((q[2 * i] + 8) & 0xF) << 4));"),
    ("q4_0: scale big-endian", "blk[0] = (uint8_t)(d & 0xFF);\n            blk[1] = (uint8_t)(d >> 8);",
     "blk[1] = (uint8_t)(d & 0xFF);\n            blk[0] = (uint8_t)(d >> 8);"),
    ("q4_0: dequantizer reads the high nibble first",
     "const int nib = (j % 2 == 0) ? (byte & 0xF) : (byte >> 4);",
     "const int nib = (j % 2 == 0) ? (byte >> 4) : (byte & 0xF);"),
    ("q4_0: dequantizer offset 7", "return oracle_f64_from_f16(d) * (double)(nib - 8);",
     "return oracle_f64_from_f16(d) * (double)(nib - 7);"),
    ("asym: matmul zero of the next group", "zeros[n * ng + k / group]);\n                double prod",
     "zeros[n * ng + (k / group + 1) % ng]);\n                double prod"),
]


@pytest.fixture(scope="module")
def workdir(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    return tmp_path_factory.mktemp("mutants")


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(workdir, name, old, new):
    src = open(oracle.SOURCE).read()
    assert src.count(old) == 1, "mutation anchor not found once: %r" % old
    mutated = src.replace(old, new)
    tag = "".join(c if c.isalnum() else "_" for c in name)
    c_path = os.path.join(str(workdir), tag + ".c")
    so_path = os.path.join(str(workdir), tag + ".so")
    with open(c_path, "w") as f:
        f.write(mutated)
    subprocess.run(["gcc", *oracle.CFLAGS, "-o", so_path, c_path, "-lm"], check=True,
                   capture_output=True)
    results = oracle_pins.run_all(oracle.Oracle(so_path))
    caught = [k for k, v in results.items() if v]
    assert caught, "mutant %r passed every pin" % name

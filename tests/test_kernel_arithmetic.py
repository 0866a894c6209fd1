"""Arithmetic identities the HIP kernels rely on, checked exhaustively on the
CPU with IEEE numpy arithmetic (no GPU, no oracle)."""
import numpy as np


def test_group_scale_product_equals_division():
    """The quantizer forms the group scale fp16_rne(a / 7) as
    fp16_rne(fp32(a) * fp32(1/7)) (one multiply instead of an IEEE fp32
    division).  For every finite fp16 absmax a both give the same fp16.  The
    right-hand side is the correctly rounded quotient: a / 7 in fp64, then
    fp16; rounding twice through 53 bits cannot change an 11-bit result."""
    bits = np.arange(0x0000, 0x7C00, dtype=np.uint16)           # +0 and every positive finite fp16
    a = bits.view(np.float16)
    product = (a.astype(np.float32) * np.float32(1.0 / 7.0)).astype(np.float16)
    quotient = (a.astype(np.float64) / 7.0).astype(np.float16)
    assert np.float32(1.0 / 7.0).view(np.uint32) == 0x3E124925
    diff = np.flatnonzero(product.view(np.uint16) != quotient.view(np.uint16))
    assert diff.size == 0, "first differing absmax: 0x%04x" % bits[diff[0]]
    # infinity and NaN map alike on both sides
    special = np.array([np.inf, np.nan], dtype=np.float16)
    p = (special.astype(np.float32) * np.float32(1.0 / 7.0)).astype(np.float16)
    assert np.isinf(p[0]) and np.isnan(p[1])


def test_group_scale_check_has_teeth():
    """The check above can fail: with 1/7 rounded to fp16 as the multiplier
    the product differs from the correctly rounded quotient for many absmax
    values.  (The fp32 multiplier has a wide margin: m / 7 for an 11-bit
    significand m repeats 001 in binary and never lies near an fp16
    rounding tie, so multipliers hundreds of fp32 ulps off still agree.)"""
    bits = np.arange(0x0001, 0x7C00, dtype=np.uint16)
    a = bits.view(np.float16).astype(np.float32)
    coarse = np.float32(np.float16(1.0 / 7.0))
    product = (a * coarse).astype(np.float16)
    quotient = (a.astype(np.float64) / 7.0).astype(np.float16)
    assert (product.view(np.uint16) != quotient.view(np.uint16)).sum() > 1000

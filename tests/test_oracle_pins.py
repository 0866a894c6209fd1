"""The oracle against its pins (CPU only)."""
import pytest

import oracle
import oracle_pins


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(orc, pin):
    fails = pin(orc)
    assert fails == [], "\n".join(fails)


def test_exact_rne_table_self_consistent():
    """The search used by the pins agrees with numpy on exact fp16 values and
    on midpoints (ties go to the even mantissa)."""
    from fractions import Fraction
    import numpy as np
    for bits in [0x0001, 0x03FF, 0x0400, 0x3C00, 0x3C01, 0x7BFF]:
        v = Fraction(float(np.uint16(bits).view(np.float16)))
        assert oracle_pins.exact_rne_f16(v) == bits
    one, nxt = Fraction(1), Fraction(float(np.uint16(0x3C01).view(np.float16)))
    assert oracle_pins.exact_rne_f16((one + nxt) / 2) == 0x3C00
    nxt2 = Fraction(float(np.uint16(0x3C02).view(np.float16)))
    assert oracle_pins.exact_rne_f16((nxt + nxt2) / 2) == 0x3C02


def test_tolerance_admits_correct_fp16_rounding():
    """The tolerance must admit the correctly rounded fp16 output for every
    exact result, including fp16's subnormal range (where the fp16 grid
    step is 2^-24 and 2^-10 |y| alone is smaller than half a step), with
    sum |x w| = |y| (one-signed terms, the tightest case).  Values one full
    fp16 step away must still fail."""
    from fractions import Fraction
    import numpy as np
    rng = np.random.default_rng(77)
    # exact results on both sides of 2^-14 and across the normal range
    exps = rng.uniform(-30.0, 15.0, 4000)
    y = np.concatenate([np.exp2(exps), -np.exp2(exps[:500]),
                        np.float64(2.0 ** -24) * rng.uniform(0.0, 1024.0, 2000)])
    for yr in y:
        bits = oracle_pins.exact_rne_f16(Fraction(float(abs(yr))))
        got = float(np.uint16(bits).view(np.float16)) * np.sign(yr)
        tol = oracle.tolerance(np.float64(yr), np.float64(abs(yr)))
        assert abs(got - yr) <= tol, (yr, got, tol)
    # a neighbour two half-steps away fails in the subnormal range
    yr = 195.57 * 2.0 ** -24
    assert abs(197 * 2.0 ** -24 - yr) > oracle.tolerance(np.float64(yr), np.float64(yr))

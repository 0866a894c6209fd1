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

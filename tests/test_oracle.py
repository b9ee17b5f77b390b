"""CPU tests: the fp64 oracle against its pins (see tests/oracle_pins.py)."""
import pytest

import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin()


def test_golden_fixture_parses():
    g = P.load_golden()
    assert g["W"].shape == (2, 3) and g["s2.dx"].shape == (2, 3)

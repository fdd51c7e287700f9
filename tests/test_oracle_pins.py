"""The fp64 oracle checked against what the KLA pages and the mathematics fix
(pins defined in tests/oracle_pins.py)."""
import pytest

import oracle
from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(oracle.fwd, oracle.decode_step)

"""The INT8 oracle against its pins (tests/q8_pins.py)."""
import pytest

import oracle.q8_oracle as Q
from tests import q8_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda p: p.__name__)
def test_q8_oracle_pin(pin):
    pin(Q)

"""The CPU oracle against library routines, closed forms, brute force and invariants."""
import pytest

import oracle.hs2_oracle as orc
from tests import oracle_pins as pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(orc)

"""The CPU oracle against its pins (no GPU).  See ``oracle_pins.py`` for what each pin checks."""
import pytest

import oracle.vp_oracle as vp_oracle
from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_oracle_pin(pin):
    pin(vp_oracle)

"""The oracle checked against hand-derived fixtures, closed forms, brute force
and a library routine (see oracle_pins.py).  CPU only."""

import pytest

from oracle import rswa_oracle as O
import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(O)

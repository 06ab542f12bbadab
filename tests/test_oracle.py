"""The float64 oracle against its pins (worked examples, closed forms,
brute force, library routines, identities); see ``oracle_pins.py``."""

import pytest

import oracle
from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(oracle)

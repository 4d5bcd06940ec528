"""The oracle against its pins (hand values, brute force, closed forms)."""

import pytest

import oracle
from tests import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle)

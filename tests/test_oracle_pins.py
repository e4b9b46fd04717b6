"""The CPU oracle against its pins (closed forms, textbook logistic, finite
differences, autograd, brute force, invariances).  No GPU."""
import pytest

import oracle
from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(oracle)

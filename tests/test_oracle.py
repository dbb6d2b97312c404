"""The CPU oracle against its pins (closed forms, library casts, brute force,
invariances, hand-derived fixtures).  No GPU."""
import pytest

import oracle
import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(oracle)

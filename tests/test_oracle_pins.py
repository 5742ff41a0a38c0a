"""The CPU oracle against its pins (see tests/pins.py for what each pin is)."""
import pytest

import oracle
import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle.default())

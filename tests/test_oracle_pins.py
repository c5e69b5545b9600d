"""The oracle against its pins (CPU only): see tests/oracle_pins.py."""
import pytest

import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin, oracle_lib):
    pin(oracle_lib)

"""The oracle against its pins (CPU only); see oracle_pins.py."""
import pytest

from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__[4:])
def test_oracle_pin(pin, oracle_lib):
    pin(oracle_lib)

"""The float64 oracle against its pins (CPU only)."""
import pytest

from tests import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(oracle_lib, pin):
    pin(oracle_lib)

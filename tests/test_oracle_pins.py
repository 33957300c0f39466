"""The fp64 oracle against its pins (CPU only)."""
import pytest

from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)

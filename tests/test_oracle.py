"""The oracle against its pins (CPU only)."""
import pytest

from oracle import attention as orc

from . import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(orc)

"""The oracle against its pins (CPU only)."""
import pytest

from oracle import rkv_oracle
import oracle_pins

pytestmark = pytest.mark.cpu


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(rkv_oracle)

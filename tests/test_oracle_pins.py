"""The float64 oracle against its pins (CPU only)."""
import pytest

from oracle import ref
from tests import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(ref)

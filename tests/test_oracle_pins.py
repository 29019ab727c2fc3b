"""The fp64 oracle against its pins (brute force, closed forms, invariants, finite differences)."""
import pytest

from tests import oracle_pins as pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin()

"""The oracle against what the pages and the mathematics fix (CPU only)."""
import pytest

from tests import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()

"""CPU pins of the oracle (see tests/pins.py for what each one fixes)."""
import pytest

from tests import pins


@pytest.mark.parametrize("pin", pins.ALL, ids=lambda f: f.__name__)
def test_pin(pin, olib):
    pin(olib)

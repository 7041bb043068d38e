"""The CPU oracle against facts fixed by the pages and by mathematics."""
import pytest

import pins



@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin_holds(pin):
    pin()

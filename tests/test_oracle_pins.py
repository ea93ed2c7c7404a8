"""The CPU oracle against its pins (torch casts, closed forms, brute force, bounds, the pages' example)."""
import pytest

import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)

"""The committed oracle against its pins (closed forms, invariants, brute
force, library special cases, format landmarks)."""
import pytest

import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)

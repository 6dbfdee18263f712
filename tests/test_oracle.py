"""The oracle against its pins (closed forms, invariants, exact-rational brute
force, independent library routines)."""
import pytest

import oracle.codecs as oc
import oracle.dsa as od
import oracle_pins as pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(od, oc)

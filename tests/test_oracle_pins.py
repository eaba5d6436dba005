"""The fp64 oracle against library routines, closed forms, exact rationals and
invariants (see oracle_pins.py for what each pin checks)."""
import pytest

import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()

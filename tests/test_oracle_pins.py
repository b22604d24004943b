"""The CPU oracle checked against closed forms, library routines, hand-derived golden
values, invariants and brute force (see ``oracle_pins.py``)."""
import pytest

import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()

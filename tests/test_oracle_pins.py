"""The fp64 oracle against its pins (hand-derived tables, trigonometric closed
values, invariants, torch float64 library routines, pure-Python brute force)."""
import pytest

import oracle_pins as P
from oracle import reference


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=[p.__name__ for p in P.ALL_PINS])
def test_oracle_pin(pin):
    pin(reference)

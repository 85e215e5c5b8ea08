"""The fp64 backward oracle against its pins (torch float64 autograd through
library routines, finite differences of the pinned forward oracle, closed
forms)."""
import pytest

import backward_pins as P
from oracle import backward


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=[p.__name__ for p in P.ALL_PINS])
def test_backward_pin(pin):
    pin(backward)

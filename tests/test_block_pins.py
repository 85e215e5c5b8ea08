"""The block-projection oracle against its pins (CPU)."""
import pytest

import block_pins as P
from oracle import block


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=[p.__name__ for p in P.ALL_PINS])
def test_block_oracle_pin(pin):
    pin(block)

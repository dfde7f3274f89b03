"""The oracle against what the pages and the mathematics fix (CPU only)."""
import pytest

import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=[p.__name__ for p in P.ALL_PINS])
def test_pin(pin):
    pin(P.real_impl())

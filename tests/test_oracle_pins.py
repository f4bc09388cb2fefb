"""The fp64 oracle against its pins (closed forms, invariants, torch's
float64 SDPA, brute force).  CPU only."""
import pytest

import oracle
from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(pin):
    pin(oracle)

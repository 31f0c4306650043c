"""The fp64 oracle against its pins (closed forms, invariants, golden hand
example, brute-force cross forms).  CPU only."""
import pytest

import oracle
from tests.oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(oracle.forward)

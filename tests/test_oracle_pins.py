"""The fp64 oracle against its pins (closed forms, invariants, golden hand
example, brute-force cross forms).  CPU only."""
import pytest

import oracle
from tests.oracle_pins import ALL_PINS, GATE_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(oracle.forward)


@pytest.mark.parametrize("pin", GATE_PINS, ids=lambda p: p.__name__)
def test_gate_pin(pin):
    pin(oracle.gate, oracle.forward)

"""The CPU oracle checked against brute force, library routines, closed forms,
invariants and the pages' structural numbers (see tests/oracle_pins.py)."""
import pytest

import oracle
from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_oracle_pin(pin):
    pin(oracle)

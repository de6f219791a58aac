"""The CPU oracle against its pins (library routines, closed forms,
invariants, brute force and the pages' worked examples)."""
import pytest

from oracle_pins import PINS


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(pin):
    pin()

"""The float64 oracle against library routines, closed forms, invariants,
exact brute force and the one-hot page-table probe (tests/oracle_pins.py)."""
import pytest

import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(orc, pin):
    pin(orc)

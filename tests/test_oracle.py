"""The CPU oracle against its pins (decode tables, exact brute force, special cases,
invariants, the worked top-k example, and the key-source equivalences)."""
import pytest

import oracle_pins as pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(oracle_lib, pin):
    pin()

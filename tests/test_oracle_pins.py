"""The CPU oracle against its pins (brute force, finite differences, closed
forms, invariants, GQA identity, decode ties).  See tests/oracle_pins.py."""
import pytest

import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(orc, pin):
    pin(orc)

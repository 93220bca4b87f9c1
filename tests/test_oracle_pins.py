"""The CPU oracle against its pins (worked expansions of the pages'
addressing, closed forms, a library routine, invariants)."""
import pytest

import oracle
from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(oracle.default())

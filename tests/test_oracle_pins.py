"""The CPU oracle against its pins (textbook routines, brute force, closed
forms and the pages' stated facts); see tests/oracle_pins.py."""
import pytest

import oracle
from tests import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(oracle)

"""Run the oracle pins (tests/oracle_pins.py) on the oracle as built."""
import pytest

from tests import oracle_pins


@pytest.mark.parametrize("check", oracle_pins.ALL_CHECKS, ids=lambda f: f.__name__[6:])
def test_oracle_pin(oracle, check):
    check(oracle)

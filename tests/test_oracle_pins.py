"""The oracle against its pins (CPU only).  See tests/oracle_pins.py."""
import pytest

from tests import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(oracle_lib, pin):
    pin(oracle_lib)

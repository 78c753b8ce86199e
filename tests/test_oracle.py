"""The fp64 oracle against facts fixed independently of its code (see oracle_pins.py)."""
import pytest

import oracle_pins as pins


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check):
    check()

"""The CPU oracle's backward pass against its pins (tests/oracle_bwd_pins.py)."""
import pytest

import oracle_bwd_pins


@pytest.mark.parametrize("pin", oracle_bwd_pins.ALL_BWD_PINS, ids=lambda f: f.__name__)
def test_bwd_pin(pin, oracle_lib):
    pin(oracle_lib)

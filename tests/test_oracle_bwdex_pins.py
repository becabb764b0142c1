"""The oracle's extended backward (grouped KV heads, band) against its pins
(tests/oracle_bwdex_pins.py)."""
import pytest

import oracle
import oracle_bwdex_pins


@pytest.mark.parametrize("pin", oracle_bwdex_pins.ALL_BWDEX_PINS, ids=lambda f: f.__name__)
def test_bwdex_pin(pin):
    pin(oracle.lib())

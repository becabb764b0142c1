"""The oracle's extended forward (grouped KV heads, band) against its pins."""
import pytest

import oracle_ex_pins


@pytest.mark.parametrize("pin", oracle_ex_pins.ALL_EX_PINS, ids=lambda f: f.__name__)
def test_ex_pin(pin, oracle_lib):
    pin(oracle_lib)

"""The CPU oracle against its pins (closed forms, invariants, library
routines, brute force, worked examples, stress classes)."""
import pytest

import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin, oracle_lib):
    pin(oracle_lib)


def test_oracle_rejects_bad_arguments(oracle_lib):
    import numpy as np
    q = np.zeros((1, 1, 4, 4), np.float32)
    with pytest.raises(RuntimeError):
        oracle_lib.attn_fwd(q, q, q, scale=1.0, rows=np.array([4], np.int32))
    with pytest.raises(RuntimeError):
        oracle_lib.attn_fwd(q, q, q, scale=1.0, rows=np.array([-1], np.int32))
    table = np.array([[0, 4]], np.int32)
    with pytest.raises(RuntimeError):
        oracle_lib.attn_fwd(q, q, q, scale=1.0, rows=table)
    with pytest.raises(ValueError):
        oracle_lib.attn_fwd(q, q, q, scale=1.0, rows=np.zeros((2, 1), np.int32))

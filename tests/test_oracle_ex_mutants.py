"""Plant plausible mistakes in copies of the oracle's extended forward (on the
CPU) and check that its pins catch every one (the oracle source itself is
never modified)."""
import pytest

import oracle
import oracle_ex_pins

MUTANTS = {
    "kv_head_modulo": ("hk = h / group;", "hk = h % Hkv;"),
    "left_edge_off_by_one": ("if (window_left >= 0 && i - window_left > lo) lo = i - window_left;",
                             "if (window_left >= 0 && i - window_left + 1 > lo) lo = i - window_left + 1;"),
    "right_edge_ignored": ("if (window_right >= 0 && (int64_t)i + window_right < hi) hi = i + window_right;\n",
                           ""),
    "causal_ignored_in_band": ("            if (causal && i < hi) hi = i;\n", ""),
    "empty_row_lse_zero": ("                lse[t] = -INFINITY;\n", "                lse[t] = 0.0;\n"),
    "band_value_from_keys": ("const float* vrow = vbh + (int64_t)j * kv_sn;",
                             "const float* vrow = kbh + (int64_t)j * kv_sn;"),
    "band_sum_skips_last": ("    for (int j = lo; j <= hi; ++j) {\n        const double w",
                            "    for (int j = lo; j < hi; ++j) {\n        const double w"),
}


@pytest.fixture(scope="module")
def source():
    with open(oracle.SOURCE) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_ex_mutant_is_caught(name, source, tmp_path):
    old, new = MUTANTS[name]
    assert source.count(old) == 1, f"mutation site for {name} not found exactly once"
    src = tmp_path / f"oracle_{name}.c"
    src.write_text(source.replace(old, new))
    lib_path = str(tmp_path / f"liboracle_{name}.so")
    oracle.build(str(src), lib_path)
    mutant = oracle.OracleLib(lib_path)
    caught = []
    for pin in oracle_ex_pins.ALL_EX_PINS:
        try:
            pin(mutant)
        except (AssertionError, RuntimeError, FloatingPointError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {name}"

"""Plant plausible mistakes in copies of the oracle's extended backward (on
the CPU) and check that its pins catch every one (the oracle source itself is
never modified)."""
import pytest

import oracle
import oracle_bwdex_pins

MUTANTS = {
    "left_edge_off_by_one": ("if (window_left >= 0 && (int64_t)i - window_left > a) a = i - window_left;",
                             "if (window_left >= 0 && (int64_t)i - window_left + 1 > a) a = i - window_left + 1;"),
    "right_edge_ignored": ("    if (window_right >= 0 && (int64_t)i + window_right < z) z = i + window_right;\n", ""),
    "causal_ignored": ("    if (causal && i < z) z = i;\n", ""),
    "stats_from_wrong_head": ("(int64_t)(hk * group + g) * q_sh + (int64_t)i * q_sn;",
                              "(int64_t)(g * Hkv + hk) * q_sh + (int64_t)i * q_sn;"),
    "row_term_without_p": ("for (int j = lo; j <= hi; ++j) D += exp(sc[j] - l) * dp[j];",
                           "for (int j = lo; j <= hi; ++j) D += dp[j];"),
    "lse_without_max": ("    const double l = top + log(z);\n", "    const double l = log(z);\n"),
    "dq_without_scale": ("for (int c = 0; c < d; ++c) out[c] = scale * out[c];", ""),
    "dk_without_scale": ("            for (int c = 0; c < d; ++c) ok[c] *= scale;\n", ""),
    "dv_from_ds": ("ov[c] += pij * (double)gi[c];", "ov[c] += dsij * (double)gi[c];"),
    "dkv_first_head_only": ("            for (int g = 0; g < group; ++g) {\n                const int h = hk * group + g;\n"
                            "                for (int i = 0; i < Nq; ++i) {",
                            "            for (int g = 0; g < 1; ++g) {\n                const int h = hk * group + g;\n"
                            "                for (int i = 0; i < Nq; ++i) {"),
    "dkv_ignores_band": ("|| j < lo || j > hi)", ")"),
    "requested_rows_not_needed": ("    for (int r = 0; dq && r < RQ; ++r) need[qrows ? qrows[r] : r] = 1;\n", ""),
}


@pytest.fixture(scope="module")
def source():
    with open(oracle.SOURCE) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_bwdex_mutant_is_caught(name, source, tmp_path):
    old, new = MUTANTS[name]
    assert source.count(old) == 1, f"mutation site for {name} not found exactly once"
    src = tmp_path / f"oracle_{name}.c"
    src.write_text(source.replace(old, new))
    lib_path = str(tmp_path / f"liboracle_{name}.so")
    oracle.build(str(src), lib_path)
    mutant = oracle.OracleLib(lib_path)
    caught = []
    for pin in oracle_bwdex_pins.ALL_BWDEX_PINS:
        try:
            pin(mutant)
        except (AssertionError, RuntimeError, FloatingPointError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {name}"

"""Plant plausible mistakes in copies of the oracle's backward pass (on the
CPU) and check that the backward pins catch every one.  The oracle source is
never modified: each mutant is a textual replacement in a temporary copy,
compiled with the same flags.

``row_term_per_block`` is the reading of [nanhubrain] "backward
recomputation" that sums the row term rowsum(P * dP) over one key block
instead of the whole row; the pins must reject it."""
import pytest

import oracle
import oracle_bwd_pins

MUTANTS = {
    "row_term_per_block": ("        D += p[j] * g[j];\n",
                           "        if (j / 4 == (vis - 1) / 4) D += p[j] * g[j];\n"),
    "dk_scale_dropped": ("            for (int c = 0; c < d; ++c) gk[c] *= scale;\n", ""),
    "ds_sign_flipped": ("const double ds = pij * (e - Dr[i]);", "const double ds = pij * (Dr[i] - e);"),
    "dv_from_ds": ("gv[c] += pij * (double)gi[c];", "gv[c] += ds * (double)gi[c];"),
    "dq_from_values": ("const float* kj = kbh + (int64_t)j * k_sn;\n                        for",
                       "const float* kj = vbh + (int64_t)j * k_sn;\n                        for"),
    "causal_column_skips_diagonal": ("for (int i = causal ? j : 0; i < Nq; ++i) {",
                                     "for (int i = causal ? j + 1 : 0; i < Nq; ++i) {"),
    "dp_from_keys": ("b += (double)gi[c] * (double)vj[c];", "b += (double)gi[c] * (double)kj[c];"),
    "lse_without_max": ("const double lse = top + log(z);", "const double lse = log(z);"),
    "dq_scale_dropped": ("for (int c = 0; c < d; ++c) out[c] *= scale;\n", ""),
}


@pytest.fixture(scope="module")
def source():
    with open(oracle.SOURCE) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_bwd_mutant_is_caught(name, source, tmp_path):
    old, new = MUTANTS[name]
    assert source.count(old) == 1, f"mutation site for {name} not found exactly once"
    src = tmp_path / f"oracle_{name}.c"
    src.write_text(source.replace(old, new))
    lib_path = str(tmp_path / f"liboracle_{name}.so")
    oracle.build(str(src), lib_path)
    mutant = oracle.OracleLib(lib_path)
    caught = []
    for pin in oracle_bwd_pins.ALL_BWD_PINS:
        try:
            pin(mutant)
        except (AssertionError, RuntimeError, FloatingPointError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {name}"

"""Plant plausible mistakes in copies of the oracle (on the CPU) and check that
the pins catch every one.  The oracle source itself is never modified: each
mutant is a textual replacement in a temporary copy, compiled with the same
flags."""
import os
import subprocess

import pytest

import oracle
import oracle_pins

MUTANTS = {
    # name: (original text, replacement)
    "exp_sign_flipped": ("double p = exp(s[j] - m);", "double p = exp(m - s[j]);"),
    "scale_dropped": ("s[j] = scale * dot;", "s[j] = dot;"),
    "value_row_from_keys": ("const float* vj = vbh + (int64_t)j * v_sn;",
                            "const float* vj = kbh + (int64_t)j * k_sn;"),
    "causal_diagonal_excluded": ("if (causal && i + 1 < nvis) nvis = i + 1;\n    if (nvis <= 0) return 0;",
                                 "if (causal && i < nvis) nvis = i;\n    if (nvis <= 0) nvis = 1;"),
    "causal_ignored": ("if (causal && i + 1 < nvis) nvis = i + 1;\n    if (nvis <= 0) return 0;",
                       "if (nvis <= 0) return 0;"),
    "lse_without_max": ("*out_lse = m + log(l);", "*out_lse = log(l);"),
    "no_normalisation": ("for (int c = 0; c < d; ++c) out_o[c] /= l;", ""),
    "min_instead_of_max": ("if (s[j] > m) m = s[j];\n    /* pass 2", "if (s[j] < m) m = s[j];\n    /* pass 2"),
    "dot_product_index": ("dot += (double)qi[c] * (double)kj[c];\n        s[j] = scale * dot;",
                          "dot += (double)qi[c] * (double)kj[0];\n        s[j] = scale * dot;"),
    "query_row_off_by_one": ("int i = rows ? rows[(rows_per_head ? bh * R : 0) + r] : r;",
                             "int i = rows ? rows[(rows_per_head ? bh * R : 0) + r] : (r + 1) % Nq;"),
    "sum_misses_first_key": ("        l += p;\n", "        if (j > 0) l += p;\n"),
    "head_stride_swapped": ("const float* kbh = k + b * k_sb + h * k_sh;",
                            "const float* kbh = k + b * k_sb + h * k_sn;"),
}


@pytest.fixture(scope="module")
def source():
    with open(oracle.SOURCE) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, source, tmp_path):
    old, new = MUTANTS[name]
    assert source.count(old) == 1, f"mutation site for {name} not found exactly once"
    src = tmp_path / f"oracle_{name}.c"
    src.write_text(source.replace(old, new))
    lib_path = str(tmp_path / f"liboracle_{name}.so")
    oracle.build(str(src), lib_path)
    mutant = oracle.OracleLib(lib_path)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(mutant)
        except (AssertionError, RuntimeError, FloatingPointError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {name}"

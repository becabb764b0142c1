"""Host model of the transposing row store (no GPU).

`store_acc_rows` (exact_attention_112_amd/csrc/fa_common.h) writes a wave's
d x 32 accumulator as rows of the output.  Lane l = 32*hi + col holds
acc[db][r] = out[col][db*32 + (r/4)*8 + hi*4 + r%4].  For each db and each
pair of adjacent register groups (gp), one v_permlane16_swap per word trades
lanes 16..31 and 48..63 of the first register set with lanes 0..15 and 32..47
of the second; then lane (col, hi) stores four words of the first set to row
col % 16 and four of the second to row col % 16 + 16, at column
db*32 + gp*16 + (col // 16)*8 + hi*4.  This restates that arithmetic lane by
lane and checks that every element of the 32 rows lands in its own place
exactly once, that each store instruction writes 64 contiguous, 64-byte
aligned bytes into each of 16 rows, and that rows at or past n_rows are left
alone.  A model with the swap's direction reversed is shown to fail.
"""
import numpy as np
import pytest

LANES = 64


def permlane16_swap(a, b):
    """(a, b) after v_permlane16_swap: lanes 16-31, 48-63 of a <-> lanes 0-15, 32-47 of b."""
    a, b = a.copy(), b.copy()
    for base in (0, 32):
        hi_a = a[base + 16:base + 32].copy()
        a[base + 16:base + 32] = b[base:base + 16]
        b[base:base + 16] = hi_a
    return a, b


def accumulator(out, d):
    """acc[db][r][lane] of the MFMA layout for a 32 x d tile `out`."""
    acc = np.zeros((d // 32, 16, LANES), dtype=out.dtype)
    for lane in range(LANES):
        col, hi = lane % 32, lane // 32
        for db in range(d // 32):
            for r in range(16):
                acc[db, r, lane] = out[col, db * 32 + (r // 4) * 8 + hi * 4 + r % 4]
    return acc


def model_store(acc, d, n_rows, swap=permlane16_swap):
    """The rows the kernel writes: dict (row, column) -> value, and the stores' byte runs."""
    written = {}
    runs = []   # per store instruction: {row: sorted columns}
    for db in range(d // 32):
        for gp in range(2):
            x = [acc[db, 8 * gp + w].copy() for w in range(4)]
            y = [acc[db, 8 * gp + 4 + w].copy() for w in range(4)]
            for w in range(4):
                x[w], y[w] = swap(x[w], y[w])
            for regs, row_off in ((x, 0), (y, 16)):
                inst = {}
                for lane in range(LANES):
                    col, hi = lane % 32, lane // 32
                    row = col % 16 + row_off
                    if row >= n_rows:
                        continue
                    dd = db * 32 + gp * 16 + (col // 16) * 8 + hi * 4
                    for w in range(4):
                        key = (row, dd + w)
                        assert key not in written, f"element {key} written twice"
                        written[key] = regs[w][lane]
                    inst.setdefault(row, []).extend(range(dd, dd + 4))
                runs.append({r: sorted(c) for r, c in inst.items()})
    return written, runs


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("n_rows", [32, 40, 31, 17, 16, 1, 0, -3])
def test_every_element_lands_once_in_its_place(d, n_rows):
    rng = np.random.default_rng(d * 100 + n_rows + 7)
    out = rng.standard_normal((32, d)).astype(np.float32)
    written, _ = model_store(accumulator(out, d), d, n_rows)
    rows = max(0, min(32, n_rows))
    assert set(written) == {(r, c) for r in range(rows) for c in range(d)}
    for (r, c), v in written.items():
        assert v == out[r, c]


@pytest.mark.parametrize("d", [64, 128])
def test_each_store_writes_64_contiguous_aligned_bytes_per_row(d):
    out = np.arange(32 * d, dtype=np.float32).reshape(32, d)
    _, runs = model_store(accumulator(out, d), d, 32)
    assert len(runs) == 4 * (d // 32)            # store instructions per wave
    for inst in runs:
        assert len(inst) == 16                    # 16 rows per instruction
        for cols in inst.values():
            assert len(cols) == 16                # 16 fp32 = 64 bytes
            assert cols == list(range(cols[0], cols[0] + 16))
            assert (cols[0] * 4) % 64 == 0        # 64-byte aligned


def test_model_flags_a_reversed_swap():
    # swapping the other halves (lanes 0-15 of a with 16-31 of b) misplaces
    # elements: the model must notice
    def reversed_swap(a, b):
        a, b = a.copy(), b.copy()
        for base in (0, 32):
            lo_a = a[base:base + 16].copy()
            a[base:base + 16] = b[base + 16:base + 32]
            b[base + 16:base + 32] = lo_a
        return a, b

    out = np.random.default_rng(1).standard_normal((32, 128)).astype(np.float32)
    written, _ = model_store(accumulator(out, 128), 128, 32, swap=reversed_swap)
    assert any(v != out[r, c] for (r, c), v in written.items())

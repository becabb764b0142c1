"""Host model of the block-sparse list a wave builds in LDS (no GPU).

`build_list` (exact_attention_112_amd/csrc/fa_common.h) compacts the indices
t < n of a mask row (forward and dQ: the key tiles a 256-query block marks)
or of a mask column pair (dK/dV: the query blocks that mark either column)
into a sorted list, one wave of 64 lanes at a time.  Each round covers 256
indices: lane i tests t = base + 4i + s for slots s = 0..3, and the entry's
position is the round's running count, plus the marked indices of all lower
lanes (one ballot per slot, counted below the lane by mbcnt), plus the marked
slots before it in its own lane.  Bits 12-15 of an entry are kept above the
index.  This restates that arithmetic lane by lane and checks the result is
exactly the sorted list of marked indices with their bits, for ragged
lengths (not multiples of 64 or 256), empty and full masks, and the largest
list the kernels accept (4096).
"""
import numpy as np
import pytest

LANES, SLOTS = 64, 4


def model_build_list(entry):
    """The wave's list for entries entry[0..n) (uint16 values, nonzero = marked)."""
    n = len(entry)
    out = {}
    count = 0
    for base in range(0, n, LANES * SLOTS):
        e = np.zeros((LANES, SLOTS), dtype=np.int64)
        for lane in range(LANES):
            for s in range(SLOTS):
                t = base + SLOTS * lane + s
                e[lane, s] = entry[t] if t < n else 0
        ballots = [[bool(e[lane, s]) for lane in range(LANES)] for s in range(SLOTS)]
        for lane in range(LANES):
            # count + sum over slots of mbcnt(ballot_s) = marked entries of lower lanes
            pos = count + sum(sum(ballots[s][:lane]) for s in range(SLOTS))
            for s in range(SLOTS):
                if e[lane, s]:
                    assert pos not in out, "two entries written to one position"
                    out[pos] = (base + SLOTS * lane + s) | (int(e[lane, s]) & 0xF000)
                    pos += 1
        count += sum(sum(b) for b in ballots)
    assert sorted(out) == list(range(count)), "positions must be 0 .. count-1"
    return [out[i] for i in range(count)]


def expected(entry):
    return [t | (int(v) & 0xF000) for t, v in enumerate(entry) if v]


@pytest.mark.parametrize("n", [1, 3, 63, 64, 65, 255, 256, 257, 300, 511, 512, 700, 1024, 4096])
@pytest.mark.parametrize("density", [0.0, 0.09, 0.5, 1.0])
def test_row_list_is_the_sorted_marked_tiles(n, density):
    rng = np.random.default_rng(n * 131 + int(density * 100))
    row = (rng.random(n) < density).astype(np.int64)
    assert model_build_list(row) == expected(row)


@pytest.mark.parametrize("n", [5, 64, 129, 300])
def test_column_pair_entries_keep_their_bits(n):
    # dK/dV: entry = 0x4000 if column 0 is marked, | 0x8000 if column 1 is
    rng = np.random.default_rng(n)
    c0 = rng.random(n) < 0.4
    c1 = rng.random(n) < 0.4
    entry = np.where(c0, 0x4000, 0) | np.where(c1, 0x8000, 0)
    got = model_build_list(entry)
    assert got == expected(entry)
    assert all((g & 0xFFF) < n for g in got)


def test_model_flags_a_wrong_lane_offset():
    # counting only the lower lanes of the entry's own slot (one ballot) would
    # misplace entries: the model must notice
    row = np.zeros(256, dtype=np.int64)
    row[[1, 4, 6]] = 1

    def wrong(entry):
        out, count = {}, 0
        for lane in range(LANES):
            for s in range(SLOTS):
                t = SLOTS * lane + s
                if entry[t]:
                    below = sum(1 for l2 in range(lane) if entry[SLOTS * l2 + s])
                    out.setdefault(count + below, t)
        return [out[k] for k in sorted(out)]

    assert wrong(row) != expected(row)
    assert model_build_list(row) == expected(row)

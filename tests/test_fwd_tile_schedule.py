"""Host model of the bf16 forward kernel's key-tile bookkeeping (no GPU).

The kernel (exact_attention_112_amd/csrc/fa_fwd.hip, fa_fwd_bf16_kernel) gives
each 256-query workgroup a range of 64-key tiles and runs them in three loops:
serial masked steps at the band's left edge, the pipelined unmasked loop, and
serial masked steps at the end (with a per-wave skip).  This module restates
that range arithmetic and loop structure in Python and checks, over many
shapes and bands, what the kernel relies on:

* every tile it loads lies in [t_begin, n_kt);
* every tile whose scores the pipelined step computes is whole (needs no
  mask) for every real row of the workgroup;
* every key a row sees lies in a tile its wave processes;
* when the pipelined step forms P of a tile, every real row of the wave has
  already seen a visible key (its running max is finite: the pipelined step
  has no stand-in for a max of -inf).

Band semantics (the [pwwt] "standard vs IO-aware" pre_tokens / next_tokens
window): key j is visible to query i iff i - wl <= j <= i + wr (a negative
edge is unbounded), j < Nk, and j <= i if causal.
"""
import itertools

import pytest

BC, BR, NW = 64, 256, 8


def visible_range(i, Nk, causal, wl, wr):
    """Keys row i sees: the interval [lo, hi] (empty if lo > hi)."""
    lo = max(0, i - wl) if wl >= 0 else 0
    hi = Nk - 1
    if wr >= 0:
        hi = min(hi, i + wr)
    if causal:
        hi = min(hi, i)
    return lo, hi


def normalise_band(Nq, Nk, wl, wr):
    """The C ABI's edge normalisation: an edge beyond every key is unbounded."""
    if wl >= Nq:
        wl = -1
    if wr >= Nk:
        wr = -1
    return wl, wr


def workgroup_plan(Nq, Nk, causal, wl, wr, qt, band):
    """Tile ranges of one workgroup, as the kernel computes them."""
    q_wg0 = qt * BR
    kv_end = min(Nk, min(q_wg0 + BR, Nq)) if causal else Nk
    n_kt = (kv_end + BC - 1) // BC
    n_full = Nk // BC
    if causal:
        n_full = min(n_full, (q_wg0 + 1) // BC)
    n_full = min(n_full, n_kt)
    t_begin = t_full_lo = 0
    n_kt_wave = []
    for w in range(NW):
        q_w0 = q_wg0 + 32 * w
        n_kt_wave.append(min(n_kt, (q_w0 + 31) // BC + 1) if causal else n_kt)
    if band:
        big = 1 << 30
        q_last = min(q_wg0 + BR, Nq) - 1
        key_lo = max(0, q_wg0 - wl) if wl >= 0 else 0
        key_hi = min(Nk - 1, q_last + wr if wr >= 0 else big)
        if causal:
            key_hi = min(key_hi, q_last)
        x_hi = min(Nk - 1, q_wg0 + wr if wr >= 0 else big)
        if causal:
            x_hi = min(x_hi, q_wg0)
        full_lo = max(0, (q_last - wl + BC - 1) // BC) if wl >= 0 else 0
        if key_lo > key_hi:
            t_begin = n_kt = n_full = t_full_lo = 0
        else:
            t_begin = key_lo // BC
            n_kt = key_hi // BC + 1
            t_full_lo = min(n_kt, max(t_begin, full_lo))
            n_full = max(t_full_lo, min(n_kt, (x_hi + 1) // BC))
        n_kt_wave = []
        for w in range(NW):
            q_w0 = q_wg0 + 32 * w
            w_hi = min(Nk - 1, q_w0 + 31 + wr if wr >= 0 else big)
            if causal:
                w_hi = min(w_hi, q_w0 + 31)
            n_kt_wave.append(min(n_kt, w_hi // BC + 1))
    return dict(q_wg0=q_wg0, n_kt=n_kt, n_full=n_full, t_begin=t_begin, t_full_lo=t_full_lo,
                n_kt_wave=n_kt_wave)


def run_schedule(plan, band, old_left_edge=False):
    """The kernel's loop structure.  Returns the steps as (kind, j, waves):
    'first' computes the scores of tile t_begin (masked unless whole);
    'left' (the band's left-edge and stage-parity steps, every wave) forms
    P_j and the masked scores of tile j+1; 'pipe' forms P_j and the unmasked
    scores of tile j+1; 'tail' forms P_j and, for a wave that needs it, the
    masked scores of tile j+1.  Also returns the tiles whose loads were
    issued.  ``old_left_edge`` replays the earlier left-edge loop, which
    stopped at the last masked tile."""
    n_kt, n_full, t_begin, t_full_lo = plan["n_kt"], plan["n_full"], plan["t_begin"], plan["t_full_lo"]
    nkw = plan["n_kt_wave"]
    allw = tuple(range(NW))
    steps, loads = [], set()
    if not band or n_kt > 0:
        loads.update({t_begin} | ({t_begin + 1} if t_begin + 1 < n_kt else set()))
        steps.append(("first", t_begin, allw))

    def top(j):
        if j + 2 < n_kt:
            loads.add(j + 2)
        if j + 1 < n_kt:
            loads.add(j + 1)

    j = t_begin
    if band:
        # masked left-edge tiles, serial, until tile j itself is whole for
        # every row (or no tile is left); then one more serial step if needed
        # so that the pipelined loop starts on stage 0
        while (j + 1 < t_full_lo) if old_left_edge else (j < t_full_lo and j + 1 < n_kt):
            top(j)
            steps.append(("left", j, allw))
            j += 1
        if ((j - t_begin) & 1) and j + 1 < n_full:
            top(j)
            steps.append(("left", j, allw))
            j += 1
    while j + 2 < n_full:
        for jj in (j, j + 1):
            top(jj)
            steps.append(("pipe", jj, allw))
        j += 2
    while j < n_kt:
        top(j)
        steps.append(("tail", j, tuple(w for w in range(NW) if j < nkw[w])))
        j += 1
    return steps, loads


def check_workgroup(Nq, Nk, causal, wl, wr, qt, old_left_edge=False):
    band = wl >= 0 or wr >= 0
    plan = workgroup_plan(Nq, Nk, causal, wl, wr, qt, band)
    steps, loads = run_schedule(plan, band, old_left_edge)
    n_kt, t_begin, nkw = plan["n_kt"], plan["t_begin"], plan["n_kt_wave"]
    q_wg0 = plan["q_wg0"]
    rows = range(q_wg0, min(q_wg0 + BR, Nq))
    where = f"Nq={Nq} Nk={Nk} causal={causal} window=({wl},{wr}) qt={qt}"
    for t in loads:
        assert t_begin <= t < n_kt, f"{where}: load of tile {t} outside [{t_begin}, {n_kt})"

    rng = {i: visible_range(i, Nk, causal, wl, wr) for i in rows}

    def whole(t, i):
        lo, hi = rng[i]
        return lo <= t * BC and (t + 1) * BC - 1 <= hi

    def sees_any(i, tiles):
        lo, hi = rng[i]
        return any(lo <= hi and lo <= (t + 1) * BC - 1 and t * BC <= hi for t in tiles)

    scored = {w: [] for w in range(NW)}    # tiles each wave has scored, in order
    formed = {w: set() for w in range(NW)}  # tiles each wave has formed P of
    for kind, j, waves in steps:
        if kind == "first":
            for w in waves:
                scored[w].append(j)
            continue
        for w in waves:
            assert scored[w] and scored[w][-1] == j, f"{where}: wave {w} forms P of tile {j} without its scores"
            formed[w].add(j)
        if kind == "pipe":
            for i in rows:
                assert whole(j + 1, i), f"{where}: pipelined step scores tile {j + 1} unmasked, row {i} sees it in part"
                assert sees_any(i, scored[i // 32 - qt * NW]), \
                    f"{where}: row {i} has no visible key when the pipelined step forms P of tile {j}"
        for w in waves:
            if kind != "tail" or j + 1 < nkw[w]:
                scored[w].append(j + 1)
    # every key a row sees lies in a tile its wave formed P of
    for i in rows:
        lo, hi = rng[i]
        for t in range(lo // BC, hi // BC + 1) if lo <= hi else ():
            assert t in formed[i // 32 - qt * NW], f"{where}: row {i} sees keys of tile {t}, which its wave skips"


SHAPES = [(1, 1), (63, 63), (64, 64), (65, 65), (255, 300), (256, 256), (257, 200), (700, 650),
          (1089, 1089), (1100, 900), (4161, 4161), (5000, 5000), (2113, 2113)]
BANDS = [(-1, -1), (0, 0), (5, -1), (63, -1), (64, -1), (100, 3), (127, 0), (255, -1), (256, 40), (512, -1),
         (1024, -1), (4095, -1), (575, -1), (1087, 5), (-1, 0), (-1, 70), (300, 300), (1000, 17)]


@pytest.mark.parametrize("Nq,Nk", SHAPES)
def test_tile_schedule(Nq, Nk):
    for (wl, wr), causal in itertools.product(BANDS, (False, True)):
        wl2, wr2 = normalise_band(Nq, Nk, wl, wr)
        for qt in range((Nq + BR - 1) // BR):
            check_workgroup(Nq, Nk, causal, wl2, wr2, qt)


def test_model_flags_the_old_left_edge_loop():
    """The left-edge loop used to stop at the last masked tile; with an even
    stage parity the pipelined step then formed P of that masked tile, whose
    running max is -inf for a row that has seen no key yet (NaN in O).  At
    Nq = Nk = 1089, causal, window (512, -1) that is row 1088 of the last
    workgroup; the model flags the old schedule there and passes the new."""
    with pytest.raises(AssertionError, match="row 1088 has no visible key"):
        check_workgroup(1089, 1089, True, 512, -1, 4, old_left_edge=True)
    with pytest.raises(AssertionError, match="row 4160 has no visible key"):
        check_workgroup(4161, 4161, True, 1024, -1, 16, old_left_edge=True)
    check_workgroup(1089, 1089, True, 512, -1, 4)
    check_workgroup(4161, 4161, True, 1024, -1, 16)

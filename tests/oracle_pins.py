"""Checks that pin the CPU oracle to facts other than itself.

Each ``pin_*`` function takes an ``oracle.OracleLib`` and raises AssertionError
when the library disagrees with what the pages and the mathematics fix.  They
are run against the real oracle (tests/test_oracle_pins.py) and against copies
of it with planted mistakes (tests/test_oracle_mutants.py), which must each
fail at least one pin.

What pins what:
* closed forms -- all-ones input (the regression class of [nanhubrain]
  "numeric safety"), identical keys / scale 0 (uniform weights: mean of the
  visible V rows), one dominant key (selects its V row), Nk = 1, causal row 0;
* invariants -- adding the same vector to every key leaves O unchanged and
  shifts LSE by scale*q.u; permuting keys and values together (non-causal)
  changes nothing; rows of P sum to 1 ([nanhubrain] "online softmax
  mathematics", the max-subtracted softmax);
* library routines -- torch's CPU scaled_dot_product_attention in float64 for
  O (its causal flag is the same top-left lower-triangular mask as [ascendai]
  section 6.1) and scipy.special.logsumexp for LSE;
* brute force -- Python Decimal at 50 digits with the unshifted exponential,
  on tiny shapes;
* hand-derived worked examples in tests/golden/worked_examples.json;
* the stress classes of [nanhubrain] "numeric safety" (all-ones, large random
  values, alternating extremes) stay finite and agree with brute force.
"""
from __future__ import annotations

import decimal
import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _bhnd(x, layout):
    """Storage-order array -> [B,H,N,d] view."""
    return x if layout == "BHND" else x.transpose(0, 2, 1, 3)


def _to_layout(x_bhnd, layout):
    return np.ascontiguousarray(x_bhnd if layout == "BHND" else x_bhnd.transpose(0, 2, 1, 3))


def _rand_case(seed, B, H, Nq, Nk, d, sigma=1.0, grid=None):
    g = _rng(seed)
    shp_q, shp_k = (B, H, Nq, d), (B, H, Nk, d)
    if grid is not None:
        # values on a dyadic grid: sums of few of them are exact in float32
        q = g.integers(-grid, grid + 1, size=shp_q).astype(np.float32) / np.float32(8)
        k = g.integers(-grid, grid + 1, size=shp_k).astype(np.float32) / np.float32(8)
        v = g.integers(-grid, grid + 1, size=shp_k).astype(np.float32) / np.float32(8)
    else:
        q = (g.standard_normal(shp_q) * sigma).astype(np.float32)
        k = (g.standard_normal(shp_k) * sigma).astype(np.float32)
        v = g.standard_normal(shp_k).astype(np.float32)
    return q, k, v


def _vis(i, Nk, causal):
    return min(Nk, i + 1) if causal else Nk


# ---------------------------------------------------------------------------
# library routines

def pin_torch_sdpa(lib):
    import torch
    import scipy.special
    cases = [
        (1, 1, 5, 5, 4, False, "BHND"),
        (2, 3, 17, 33, 8, False, "BSND"),
        (1, 2, 33, 33, 16, True, "BHND"),
        (2, 2, 40, 24, 8, True, "BSND"),   # causal, Nq > Nk: rows >= Nk see every key
        (1, 2, 24, 40, 8, True, "BHND"),   # causal, Nq < Nk: top-left alignment
        (1, 1, 7, 1, 4, False, "BHND"),
        (1, 1, 64, 64, 64, True, "BSND"),
    ]
    for n, (B, H, Nq, Nk, d, causal, layout) in enumerate(cases):
        q, k, v = _rand_case(100 + n, B, H, Nq, Nk, d)
        scale = 1.0 / math.sqrt(d) if n % 2 == 0 else 0.37
        o, lse = lib.attn_fwd(_to_layout(q, layout), _to_layout(k, layout), _to_layout(v, layout),
                              scale=scale, causal=causal, layout=layout)
        tq, tk, tv = (torch.from_numpy(x.astype(np.float64)) for x in (q, k, v))
        ref = torch.nn.functional.scaled_dot_product_attention(
            tq, tk, tv, is_causal=causal, scale=scale).numpy()
        err = np.abs(o - ref).max()
        assert err < 1e-12, f"O vs torch sdpa, case {n}: {err}"
        s = scale * np.einsum("bhid,bhjd->bhij", q.astype(np.float64), k.astype(np.float64))
        if causal:
            s = np.where(np.arange(Nk)[None, :] > np.arange(Nq)[:, None], -np.inf, s)
        ref_lse = scipy.special.logsumexp(s, axis=-1)
        err = np.abs(lse - ref_lse).max()
        assert err < 1e-12, f"LSE vs scipy logsumexp, case {n}: {err}"


# ---------------------------------------------------------------------------
# brute force in Decimal, no max shift

def _decimal_attn(q, k, v, scale, causal):
    ctx = decimal.Context(prec=50)
    D = decimal.Decimal
    Nq, d = q.shape
    Nk = k.shape[0]
    sc = D(float(scale))
    o = np.zeros((Nq, d))
    lse = np.zeros(Nq)
    for i in range(Nq):
        nv = _vis(i, Nk, causal)
        w = []
        for j in range(nv):
            dot = sum((D(float(q[i, c])) * D(float(k[j, c])) for c in range(d)), D(0))
            w.append(ctx.exp(ctx.multiply(sc, dot)))
        z = sum(w, D(0))
        for c in range(d):
            num = sum((w[j] * D(float(v[j, c])) for j in range(nv)), D(0))
            o[i, c] = float(ctx.divide(num, z))
        lse[i] = float(ctx.ln(z))
    return o, lse


def pin_decimal_bruteforce(lib):
    for n, (Nq, Nk, d, causal, sigma) in enumerate([
            (3, 4, 2, False, 1.0), (5, 5, 3, True, 1.0), (4, 7, 4, True, 2.0),
            (6, 3, 8, False, 3.0), (2, 9, 5, False, 0.5)]):
        q, k, v = _rand_case(200 + n, 1, 1, Nq, Nk, d, sigma=sigma)
        scale = 0.7
        o, lse = lib.attn_fwd(q, k, v, scale=scale, causal=causal)
        ro, rl = _decimal_attn(q[0, 0], k[0, 0], v[0, 0], scale, causal)
        assert np.abs(o[0, 0] - ro).max() < 1e-12, f"O vs Decimal brute force, case {n}"
        assert np.abs(lse[0, 0] - rl).max() < 1e-12, f"LSE vs Decimal brute force, case {n}"


# ---------------------------------------------------------------------------
# closed forms

def pin_all_ones(lib):
    """Q = K = V = 1: every visible score is scale*d, O = 1 exactly,
    LSE = scale*d + ln|Vis(i)|."""
    for causal in (False, True):
        for (Nq, Nk, d) in ((8, 8, 4), (5, 12, 16), (12, 5, 8)):
            q = np.ones((1, 2, Nq, d), np.float32)
            k = np.ones((1, 2, Nk, d), np.float32)
            scale = 1.0 / math.sqrt(d)
            o, lse = lib.attn_fwd(q, k, k.copy(), scale=scale, causal=causal)
            assert np.abs(o - 1.0).max() < 1e-14, "all-ones: O must be 1"
            for i in range(Nq):
                exp_lse = scale * d + math.log(_vis(i, Nk, causal))
                assert abs(lse[0, 0, i] - exp_lse) < 1e-13, f"all-ones LSE row {i}"


def pin_uniform(lib):
    """Identical keys, or scale 0: uniform weights over the visible keys, so O
    is the mean (causal: prefix mean) of V; LSE = s + ln|Vis(i)|."""
    B, H, Nq, Nk, d = 1, 2, 9, 9, 4
    q, _, v = _rand_case(300, B, H, Nq, Nk, d)
    krow = _rng(301).standard_normal(d).astype(np.float32)
    k = np.broadcast_to(krow, (B, H, Nk, d)).copy()
    for causal in (False, True):
        o, lse = lib.attn_fwd(q, k, v, scale=0.5, causal=causal)
        for h in range(H):
            for i in range(Nq):
                nv = _vis(i, Nk, causal)
                mean = v[0, h, :nv].astype(np.float64).mean(axis=0)
                assert np.abs(o[0, h, i] - mean).max() < 1e-13, f"identical keys row {i}"
                s = 0.5 * float(np.dot(q[0, h, i].astype(np.float64), krow.astype(np.float64)))
                assert abs(lse[0, h, i] - (s + math.log(nv))) < 1e-12
        q2, k2, v2 = _rand_case(302, B, H, Nq, Nk, d)
        o, lse = lib.attn_fwd(q2, k2, v2, scale=0.0, causal=causal)
        for i in range(Nq):
            nv = _vis(i, Nk, causal)
            mean = v2[0, :, :nv].astype(np.float64).mean(axis=1)
            assert np.abs(o[0, :, i] - mean).max() < 1e-13, "scale 0 must average V"
            assert np.abs(lse[0, :, i] - math.log(nv)).max() < 1e-13


def pin_dominant_key(lib):
    """One key whose score exceeds every other by > 60: O is its V row to
    within e^-60 relative, LSE equals its score to the same order."""
    Nq, Nk, d = 6, 10, 4
    q, k, v = _rand_case(400, 1, 1, Nq, Nk, d, grid=4)
    q[0, 0] = np.abs(q[0, 0]) + np.float32(1)           # every query positive
    jstar = 6
    k[0, 0, jstar] = np.float32(64.0)                   # its score >= 64*4*1 = 256
    scale = 1.0
    o, lse = lib.attn_fwd(q, k, v, scale=scale, causal=False)
    for i in range(Nq):
        s = q[0, 0, i].astype(np.float64) @ k[0, 0].astype(np.float64).T
        assert s[jstar] - np.delete(s, jstar).max() > 60
        assert np.abs(o[0, 0, i] - v[0, 0, jstar]).max() < 1e-15
        assert abs(lse[0, 0, i] - s[jstar]) < 1e-12 * abs(s[jstar])


def pin_single_key_and_causal_row0(lib):
    """Nk = 1: O = V[0], LSE = scale*q.k0.  Causal: row 0 sees only key 0."""
    q, k, v = _rand_case(500, 2, 3, 7, 1, 8)
    o, lse = lib.attn_fwd(q, k, v, scale=0.3, causal=False)
    assert np.abs(o - v.astype(np.float64)).max() < 1e-15
    s = 0.3 * np.einsum("bhid,bhd->bhi", q.astype(np.float64), k[:, :, 0].astype(np.float64))
    assert np.abs(lse - s).max() < 1e-13
    q, k, v = _rand_case(501, 2, 3, 7, 7, 8)
    o, lse = lib.attn_fwd(q, k, v, scale=0.3, causal=True)
    assert np.abs(o[:, :, 0] - v[:, :, 0].astype(np.float64)).max() < 1e-15
    s0 = 0.3 * np.einsum("bhd,bhd->bh", q[:, :, 0].astype(np.float64), k[:, :, 0].astype(np.float64))
    assert np.abs(lse[:, :, 0] - s0).max() < 1e-13


# ---------------------------------------------------------------------------
# invariants

def pin_key_shift(lib):
    """K + 1 u^T: scores of row i all shift by scale*q_i.u, so O is unchanged and
    LSE shifts by scale*q_i.u.  Values on a dyadic grid keep K+u exact."""
    for causal in (False, True):
        q, k, v = _rand_case(600, 1, 2, 11, 13, 8, grid=8)
        u = (_rng(601).integers(-8, 9, size=8).astype(np.float32) / np.float32(8))
        k2 = k + u
        assert np.array_equal(k2 - u, k)
        scale = 0.25
        o1, l1 = lib.attn_fwd(q, k, v, scale=scale, causal=causal)
        o2, l2 = lib.attn_fwd(q, k2, v, scale=scale, causal=causal)
        shift = scale * (q.astype(np.float64) @ u.astype(np.float64))
        assert np.abs(o1 - o2).max() < 1e-13, "key shift must leave O unchanged"
        assert np.abs((l2 - l1) - shift).max() < 1e-12, "key shift must shift LSE by scale*q.u"


def pin_permutation(lib):
    """Non-causal: permuting keys and values together changes nothing."""
    q, k, v = _rand_case(700, 2, 2, 9, 15, 8)
    perm = _rng(701).permutation(15)
    o1, l1 = lib.attn_fwd(q, k, v, scale=0.4)
    o2, l2 = lib.attn_fwd(q, k[:, :, perm].copy(), v[:, :, perm].copy(), scale=0.4)
    assert np.abs(o1 - o2).max() < 1e-13 and np.abs(l1 - l2).max() < 1e-13


def pin_probs_normalised(lib):
    """Rows of P sum to 1, masked entries are exactly 0, P >= 0, and
    P_ij = exp(s_ij - LSE_i) (the recomputation identity)."""
    for causal in (False, True):
        q, k, v = _rand_case(800, 1, 1, 12, 12, 8, sigma=2.0)
        p = lib.attn_probs(q[0, 0], k[0, 0], scale=0.5, causal=causal)
        assert np.abs(p.sum(axis=1) - 1).max() < 1e-14
        assert (p >= 0).all()
        if causal:
            assert (p[np.triu_indices(12, 1)] == 0).all()
        _, lse = lib.attn_fwd(q, k, v, scale=0.5, causal=causal)
        s = 0.5 * (q[0, 0].astype(np.float64) @ k[0, 0].astype(np.float64).T)
        rec = np.exp(s - lse[0, 0][:, None])
        if causal:
            rec = np.tril(rec)
        assert np.abs(rec - p).max() < 1e-13


def pin_rows_subset(lib):
    """The row-sampled mode returns exactly the sampled rows of the full run."""
    for layout in ("BHND", "BSND"):
        q, k, v = _rand_case(900, 2, 3, 20, 20, 8)
        q, k, v = (_to_layout(x, layout) for x in (q, k, v))
        rows = np.array([0, 3, 4, 19], np.int32)
        for causal in (False, True):
            of, lf = lib.attn_fwd(q, k, v, scale=0.3, causal=causal, layout=layout)
            os_, ls = lib.attn_fwd(q, k, v, scale=0.3, causal=causal, layout=layout, rows=rows)
            assert np.array_equal(of[:, :, rows], os_) and np.array_equal(lf[:, :, rows], ls)


def pin_row_table(lib):
    """A row table (rows of their own for each head) returns, for every head,
    exactly its rows of the full run, in the table's order."""
    for layout in ("BHND", "BSND"):
        q, k, v = _rand_case(901, 2, 3, 20, 23, 8)
        q, k, v = (_to_layout(x, layout) for x in (q, k, v))
        g = _rng(902)
        table = np.stack([g.permutation(20)[:5] for _ in range(6)]).astype(np.int32)
        for causal in (False, True):
            of, lf = lib.attn_fwd(q, k, v, scale=0.3, causal=causal, layout=layout)
            ot, lt = lib.attn_fwd(q, k, v, scale=0.3, causal=causal, layout=layout, rows=table)
            for bh in range(6):
                b, h = divmod(bh, 3)
                assert np.array_equal(of[b, h, table[bh]], ot[b, h]) and np.array_equal(lf[b, h, table[bh]], lt[b, h])


# ---------------------------------------------------------------------------
# worked examples

def load_worked_examples():
    with open(os.path.join(GOLDEN, "worked_examples.json")) as f:
        return json.load(f)["cases"]


def pin_worked_examples(lib):
    for case in load_worked_examples():
        q = np.array(case["q"], np.float32)[None, None]
        k = np.array(case["k"], np.float32)[None, None]
        v = np.array(case["v"], np.float32)[None, None]
        o, lse = lib.attn_fwd(q, k, v, scale=case["scale"], causal=case["causal"])
        exp_o = np.array([[eval(e, {"math": math}) for e in row] for row in case["o"]])
        exp_l = np.array([eval(e, {"math": math}) for e in case["lse"]])
        assert np.abs(o[0, 0] - exp_o).max() < 1e-14, case["name"]
        assert np.abs(lse[0, 0] - exp_l).max() < 1e-14, case["name"]


# ---------------------------------------------------------------------------
# stress classes ([nanhubrain] "numeric safety")

def pin_stress_classes(lib):
    # large random values: scores reach several hundred, exp() of them overflows
    # double unless the maximum is subtracted first
    q, k, v = _rand_case(1000, 1, 1, 5, 6, 4, sigma=30.0)
    o, lse = lib.attn_fwd(q, k, v, scale=1.0)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    ro, rl = _decimal_attn(q[0, 0], k[0, 0], v[0, 0], 1.0, False)
    assert np.abs(o[0, 0] - ro).max() < 1e-12 and np.abs(lse[0, 0] - rl).max() < 1e-9
    # alternating extremes: query rows alternate +-big, keys alternate sign
    d = 4
    q = np.array([[[[(-1) ** i * 40.0] * d for i in range(6)]]], np.float32)
    k = np.array([[[[(-1) ** j * 3.0] * d for j in range(7)]]], np.float32)
    v = _rand_case(1001, 1, 1, 7, 7, d)[2]
    for causal in (False, True):
        o, lse = lib.attn_fwd(q, k, v, scale=1.0, causal=causal)
        assert np.isfinite(o).all() and np.isfinite(lse).all()
        ro, rl = _decimal_attn(q[0, 0], k[0, 0], v[0, 0], 1.0, causal)
        assert np.abs(o[0, 0] - ro).max() < 1e-12 and np.abs(lse[0, 0] - rl).max() < 1e-9


ALL_PINS = [
    pin_torch_sdpa, pin_decimal_bruteforce, pin_all_ones, pin_uniform, pin_dominant_key,
    pin_single_key_and_causal_row0, pin_key_shift, pin_permutation, pin_probs_normalised,
    pin_rows_subset, pin_row_table, pin_worked_examples, pin_stress_classes,
]

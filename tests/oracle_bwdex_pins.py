"""Checks that pin the oracle's extended backward (grouped KV heads, band of
visible keys) to facts other than itself.

Each ``pin_*`` takes an ``oracle.OracleLib`` and raises AssertionError on a
disagreement.  Run against the real oracle (tests/test_oracle_bwdex_pins.py)
and against copies with planted mistakes (tests/test_oracle_bwdex_mutants.py).

What pins what:
* a library routine -- torch's autograd through its CPU
  scaled_dot_product_attention in float64, with the band (and causal) as an
  explicit boolean mask and the KV heads repeated per group
  (torch.repeat_interleave), whose gradient with respect to the repeated
  heads is summed back over each group;
* the plain backward -- with Hkv = H and no band it must equal the pinned
  oracle_attn_bwd;
* closed forms -- window (0, 0): each query sees only key i, so P = 1,
  dS = 0, dQ = dK = 0 and dV_i = the sum of dO_i over the query heads of
  the group; rows with no visible key give dQ = 0 and pass nothing on;
  causal with window (left, -1) equals window (left, 0);
* selection -- the qrows / krows arguments return the matching slices of the
  full result.
"""
from __future__ import annotations

import numpy as np

from oracle_pins import _rng, _to_layout


def _case(seed, B, H, Hkv, Nq, Nk, d):
    g = _rng(seed)
    q = g.standard_normal((B, H, Nq, d)).astype(np.float32)
    k = g.standard_normal((B, Hkv, Nk, d)).astype(np.float32)
    v = g.standard_normal((B, Hkv, Nk, d)).astype(np.float32)
    do = g.standard_normal((B, H, Nq, d)).astype(np.float32)
    return q, k, v, do


def _bwd(lib, q, k, v, do, scale, causal, window, layout="BHND", **kw):
    t = lambda x: _to_layout(x, layout)
    return lib.attn_bwd_ex(t(q), t(k), t(v), t(do), scale=scale, causal=causal, window=window,
                           layout=layout, **kw)


def _mask(Nq, Nk, causal, window):
    i = np.arange(Nq)[:, None]
    j = np.arange(Nk)[None, :]
    m = np.ones((Nq, Nk), dtype=bool)
    if window[0] >= 0:
        m &= j >= i - window[0]
    if window[1] >= 0:
        m &= j <= i + window[1]
    if causal:
        m &= j <= i
    return m


def pin_torch_autograd(lib):
    import torch
    import torch.nn.functional as F

    for seed, (B, H, Hkv, Nq, Nk, d), causal, window, layout in [
        (71, (1, 4, 2, 23, 29, 8), False, (6, 4), "BHND"),
        (72, (2, 6, 3, 20, 20, 4), True, (5, -1), "BSND"),
        (73, (1, 3, 1, 18, 30, 6), False, (-1, 3), "BHND"),
        (74, (1, 4, 4, 25, 16, 5), True, (-1, -1), "BSND"),
    ]:
        q, k, v, do = _case(seed, B, H, Hkv, Nq, Nk, d)
        scale = 1.0 / np.sqrt(d)
        m = _mask(Nq, Nk, causal, window)
        assert m.any(axis=1).all(), "pin cases keep a visible key in every row"
        dq, dk, dv = _bwd(lib, q, k, v, do, scale, causal, window, layout)
        rep = H // Hkv
        tq = torch.tensor(q, dtype=torch.float64, requires_grad=True)
        tk = torch.tensor(k, dtype=torch.float64, requires_grad=True)
        tv = torch.tensor(v, dtype=torch.float64, requires_grad=True)
        o = F.scaled_dot_product_attention(tq, tk.repeat_interleave(rep, dim=1), tv.repeat_interleave(rep, dim=1),
                                           attn_mask=torch.tensor(m), scale=scale)
        o.backward(torch.tensor(do, dtype=torch.float64))
        for name, got, want in (("dQ", dq, tq.grad), ("dK", dk, tk.grad), ("dV", dv, tv.grad)):
            err = float(np.max(np.abs(got - want.numpy())))
            assert err < 1e-11, f"{name} vs torch autograd: {err:.2e}"


def pin_reduces_to_plain(lib):
    for causal in (False, True):
        q, k, v, do = _case(75 + causal, 2, 3, 3, 27, 31, 7)
        a = _bwd(lib, q, k, v, do, 0.35, causal, (-1, -1))
        b = lib.attn_bwd(q, k, v, do, scale=0.35, causal=causal)
        for name, x, y in zip(("dQ", "dK", "dV"), a, b):
            assert np.max(np.abs(x - y)) < 1e-13, f"{name}: Hkv = H, no band must equal the plain backward"


def pin_band_closed_forms(lib):
    B, H, Hkv = 1, 4, 2
    q, k, v, do = _case(77, B, H, Hkv, 13, 9, 5)
    dq, dk, dv = _bwd(lib, q, k, v, do, 0.5, False, (0, 0))
    assert np.max(np.abs(dq)) < 1e-14 and np.max(np.abs(dk)) < 1e-14, "window (0,0): dS = 0"
    grp = H // Hkv
    for hk in range(Hkv):
        want = do[0, hk * grp:(hk + 1) * grp, :9].astype(np.float64).sum(axis=0)
        assert np.max(np.abs(dv[0, hk] - want)) < 1e-13, "window (0,0): dV_i = sum of the group's dO_i"
    # rows 9..12 see no key (Nk = 9): no gradient; their dO must not reach dV
    do2 = do.copy()
    do2[:, :, 9:] *= 3.0
    dq2, dk2, dv2 = _bwd(lib, q, k, v, do2, 0.5, False, (0, 0))
    assert np.all(dq2[:, :, 9:] == 0.0), "empty rows: dQ = 0"
    assert np.array_equal(dv, dv2) and np.array_equal(dk, dk2), "empty rows pass no gradient on"
    # causal with an unbounded right edge is the right edge 0
    q, k, v, do = _case(78, 1, 2, 1, 17, 17, 4)
    a = _bwd(lib, q, k, v, do, 0.4, True, (3, -1))
    b = _bwd(lib, q, k, v, do, 0.4, False, (3, 0))
    for x, y in zip(a, b):
        assert np.array_equal(x, y), "causal = right edge 0"


def pin_row_selection(lib):
    q, k, v, do = _case(79, 1, 4, 2, 40, 35, 6)
    full = _bwd(lib, q, k, v, do, 0.3, True, (9, -1))
    qr = np.array([39, 0, 17, 5], dtype=np.int32)
    kr = np.array([34, 2, 20], dtype=np.int32)
    sub = _bwd(lib, q, k, v, do, 0.3, True, (9, -1), qrows=qr, krows=kr)
    assert np.array_equal(sub[0], full[0][:, :, qr]), "qrows select rows of dQ"
    assert np.array_equal(sub[1], full[1][:, :, kr]), "krows select rows of dK"
    assert np.array_equal(sub[2], full[2][:, :, kr]), "krows select rows of dV"
    only_q = _bwd(lib, q, k, v, do, 0.3, True, (9, -1), qrows=qr, want_dkv=False)
    assert np.array_equal(only_q[0], full[0][:, :, qr]) and only_q[1] is None, "dQ alone"


ALL_BWDEX_PINS = [pin_torch_autograd, pin_reduces_to_plain, pin_band_closed_forms, pin_row_selection]

"""Checks that pin the oracle's extended forward (grouped KV heads, band of
visible keys) to facts other than itself.

Each ``pin_*`` takes an ``oracle.OracleLib`` and raises AssertionError on a
disagreement.  Run against the real oracle (tests/test_oracle_ex_pins.py)
and against copies with planted mistakes (tests/test_oracle_ex_mutants.py).

What pins what:
* library routines -- torch's CPU scaled_dot_product_attention in float64
  with an explicit boolean mask (the band, and causal) and the KV heads
  repeated per group (torch.repeat_interleave), and torch.logsumexp for LSE;
* the plain forward -- with Hkv = H and no band it must agree with the
  pinned plain oracle (oracle_attn_fwd);
* closed forms -- window (0, 0): each query sees only key i, so O_i = v_i
  and LSE_i = scale q_i.k_i; rows with no visible key give O = 0 and
  LSE = -inf; window (left, -1) with causal = window (left, 0);
* the head map -- one KV head per group, duplicated to H heads with Hkv = H,
  gives the same result as the grouped call.
"""
from __future__ import annotations

import numpy as np

from oracle_pins import _rng, _to_layout


def _case(seed, B, H, Hkv, Nq, Nk, d):
    g = _rng(seed)
    q = g.standard_normal((B, H, Nq, d)).astype(np.float32)
    k = g.standard_normal((B, Hkv, Nk, d)).astype(np.float32)
    v = g.standard_normal((B, Hkv, Nk, d)).astype(np.float32)
    return q, k, v


def _ex(lib, q, k, v, scale, causal, window, layout="BHND", rows=None):
    return lib.attn_fwd_ex(_to_layout(q, layout), _to_layout(k, layout), _to_layout(v, layout),
                           scale=scale, causal=causal, window=window, layout=layout, rows=rows)


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


def pin_torch_masked_sdpa(lib):
    import torch
    import torch.nn.functional as F

    for seed, (B, H, Hkv, Nq, Nk, d), causal, window, layout in [
        (51, (1, 4, 2, 37, 41, 8), False, (5, 3), "BHND"),
        (52, (2, 6, 1, 30, 30, 4), True, (7, -1), "BSND"),
        (53, (1, 3, 3, 25, 40, 6), False, (-1, 2), "BHND"),
        (54, (1, 4, 4, 50, 20, 5), True, (-1, -1), "BSND"),
    ]:
        q, k, v = _case(seed, B, H, Hkv, Nq, Nk, d)
        scale = 1.0 / np.sqrt(d)
        o, lse = _ex(lib, q, k, v, scale, causal, window, layout)
        m = _mask(Nq, Nk, causal, window)
        rep = H // Hkv
        tq = torch.tensor(q, dtype=torch.float64)
        tk = torch.tensor(k, dtype=torch.float64).repeat_interleave(rep, dim=1)
        tv = torch.tensor(v, dtype=torch.float64).repeat_interleave(rep, dim=1)
        tm = torch.tensor(m)
        want = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=tm, scale=scale).numpy()
        s = scale * (tq @ tk.transpose(-1, -2))
        want_lse = torch.logsumexp(s.masked_fill(~tm, float("-inf")), dim=-1).numpy()
        live = m.any(axis=1)
        err_o = np.max(np.abs(o[:, :, live] - want[:, :, live]))
        err_l = np.max(np.abs(lse[:, :, live] - want_lse[:, :, live]))
        assert err_o < 1e-12 and err_l < 1e-12, f"vs torch masked SDPA: O {err_o:.2e}, LSE {err_l:.2e}"
        assert np.all(o[:, :, ~live] == 0.0) and np.all(np.isneginf(lse[:, :, ~live])), "empty rows"


def pin_reduces_to_plain(lib):
    for causal in (False, True):
        q, k, v = _case(55 + causal, 2, 3, 3, 29, 33, 7)
        o, lse = _ex(lib, q, k, v, 0.3, causal, (-1, -1))
        o2, lse2 = lib.attn_fwd(q, k, v, scale=0.3, causal=causal)
        assert np.max(np.abs(o - o2)) < 1e-14 and np.max(np.abs(lse - lse2)) < 1e-14, \
            "Hkv = H, no band: must equal the plain forward oracle"


def pin_band_closed_forms(lib):
    q, k, v = _case(57, 1, 2, 1, 12, 9, 5)
    scale = 0.5
    o, lse = _ex(lib, q, k, v, scale, False, (0, 0))
    for i in range(9):      # rows with key i
        for h in range(2):
            assert np.max(np.abs(o[0, h, i] - v[0, 0, i])) < 1e-15, "window (0,0): O_i = v_i"
            want = scale * float(np.dot(q[0, h, i].astype(np.float64), k[0, 0, i].astype(np.float64)))
            assert abs(lse[0, h, i] - want) < 1e-13, "window (0,0): LSE_i = scale q_i.k_i"
    assert np.all(o[0, :, 9:] == 0.0) and np.all(np.isneginf(lse[0, :, 9:])), "rows past Nk see no key"
    # causal with an unbounded right edge is the right edge 0
    a = _ex(lib, q, k, v, scale, True, (3, -1))
    b = _ex(lib, q, k, v, scale, False, (3, 0))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]), "causal = right edge 0"
    # a band wider than the sequence changes nothing
    a = _ex(lib, q, k, v, scale, False, (100, 100))
    b = _ex(lib, q, k, v, scale, False, (-1, -1))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]), "wide band = no band"


def pin_head_map(lib):
    B, H, Hkv = 2, 6, 2
    q, k, v = _case(58, B, H, Hkv, 21, 26, 4)
    grp = H // Hkv
    for causal, window in ((False, (-1, -1)), (True, (4, -1))):
        o, lse = _ex(lib, q, k, v, 0.4, causal, window)
        kd = np.repeat(k, grp, axis=1)   # KV head of query head h is h // grp
        vd = np.repeat(v, grp, axis=1)
        o2, lse2 = _ex(lib, q, kd, vd, 0.4, causal, window)
        assert np.array_equal(o, o2) and np.array_equal(lse, lse2), "grouped heads = duplicated heads"
    # the rows argument selects rows
    rows = np.array([20, 0, 7], dtype=np.int32)
    o, lse = _ex(lib, q, k, v, 0.4, True, (4, -1))
    o3, lse3 = _ex(lib, q, k, v, 0.4, True, (4, -1), rows=rows)
    assert np.array_equal(o3, o[:, :, rows]) and np.array_equal(lse3, lse[:, :, rows]), "row subset"


ALL_EX_PINS = [pin_torch_masked_sdpa, pin_reduces_to_plain, pin_band_closed_forms, pin_head_map]

"""Checks that pin the CPU oracle's backward pass (dQ, dK, dV) to facts other
than itself.

Each ``pin_*`` function takes an ``oracle.OracleLib`` and raises AssertionError
when the library's gradients disagree with what the mathematics fixes.  They
run against the real oracle (tests/test_oracle_bwd_pins.py) and against copies
of it with planted mistakes (tests/test_oracle_bwd_mutants.py), each of which
must fail at least one pin.

What pins what:
* library routines -- torch autograd in float64 through torch's CPU
  scaled_dot_product_attention (the library's own backward of the forward
  definition, independent of the oracle's gradient formulas);
* finite differences -- central differences of the forward oracle's loss
  sum(dO * O) on dyadic inputs, whose perturbed copies are exact in float32;
* closed forms -- Nk = 1 (no gradient reaches Q or K; dV_0 = sum_i dO_i) and
  scale 0 (uniform weights: dQ = dK = 0, dV_j = sum over the queries that see
  key j of dO_i / |Vis(i)|);
* invariants -- sum_j dK_j = 0 (every row of dS sums to 0 over its visible
  keys), sum_j dV_j = sum_i dO_i (rows of P sum to 1), dQ unchanged when the
  same vector is added to every key, key/value permutation (non-causal)
  permutes dK and dV and leaves dQ, and sampled rows equal the full result.
"""
from __future__ import annotations

import numpy as np

from oracle_pins import _rng, _to_layout


def _case(seed, B, H, Nq, Nk, d, grid=None):
    g = _rng(seed)
    if grid is not None:
        mk = lambda n: (g.integers(-grid, grid + 1, size=(B, H, n, d)).astype(np.float32)
                        / np.float32(16))
    else:
        mk = lambda n: g.standard_normal((B, H, n, d)).astype(np.float32)
    return mk(Nq), mk(Nk), mk(Nk), mk(Nq)   # q, k, v, do  ([B,H,N,d])


def _bwd(lib, q, k, v, do, scale, causal, layout="BHND", **kw):
    dq, dk, dv = lib.attn_bwd(_to_layout(q, layout), _to_layout(k, layout), _to_layout(v, layout),
                              _to_layout(do, layout), scale=scale, causal=causal, layout=layout, **kw)
    return dq, dk, dv


def _close(a, b, tol, what):
    err = np.max(np.abs(a - b)) / max(1.0, np.max(np.abs(b)))
    assert err <= tol, f"{what}: relative error {err:.3e} > {tol:.1e}"


def pin_torch_autograd(lib):
    import torch
    import torch.nn.functional as F

    for seed, (B, H, Nq, Nk, d), causal, layout in [
        (11, (2, 2, 13, 11, 5), False, "BHND"),
        (12, (1, 3, 11, 17, 8), True, "BSND"),
        (13, (1, 1, 33, 33, 4), True, "BHND"),
    ]:
        q, k, v, do = _case(seed, B, H, Nq, Nk, d)
        scale = 1.0 / np.sqrt(d)
        tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
        o = F.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
        (o * torch.tensor(do, dtype=torch.float64)).sum().backward()
        dq, dk, dv = _bwd(lib, q, k, v, do, scale, causal, layout)
        _close(dq, tq.grad.numpy(), 1e-10, "dQ vs torch autograd")
        _close(dk, tk.grad.numpy(), 1e-10, "dK vs torch autograd")
        _close(dv, tv.grad.numpy(), 1e-10, "dV vs torch autograd")


def pin_finite_differences(lib):
    B, H, Nq, Nk, d = 1, 1, 5, 4, 3
    h = 2.0 ** -10
    for causal in (False, True):
        q, k, v, do = _case(21 + causal, B, H, Nq, Nk, d, grid=24)
        scale = 0.75

        def loss(qq, kk, vv):
            o, _ = lib.attn_fwd(qq, kk, vv, scale=scale, causal=causal)
            return float(np.sum(o * do.astype(np.float64)))

        dq, dk, dv = _bwd(lib, q, k, v, do, scale, causal)
        for name, x, grad in (("dQ", q, dq), ("dK", k, dk), ("dV", v, dv)):
            fd = np.zeros(x.shape)
            for idx in np.ndindex(*x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += np.float32(h)
                xm[idx] -= np.float32(h)
                args_p = [q, k, v]
                args_m = [q, k, v]
                pos = {"dQ": 0, "dK": 1, "dV": 2}[name]
                args_p[pos], args_m[pos] = xp, xm
                fd[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
            _close(grad, fd, 1e-5, f"{name} vs central differences (causal={causal})")


def pin_closed_forms(lib):
    # Nk = 1: P = 1, dS = 0
    q, k, v, do = _case(31, 2, 2, 6, 1, 4)
    for causal in (False, True):
        dq, dk, dv = _bwd(lib, q, k, v, do, 0.5, causal)
        assert np.max(np.abs(dq)) < 1e-14 and np.max(np.abs(dk)) < 1e-14, "Nk=1: dQ, dK must vanish"
        _close(dv[:, :, 0], do.astype(np.float64).sum(axis=2), 1e-13, "Nk=1: dV_0 = sum_i dO_i")
    # scale 0: uniform weights over the visible keys
    q, k, v, do = _case(32, 1, 2, 7, 9, 3)
    for causal in (False, True):
        dq, dk, dv = _bwd(lib, q, k, v, do, 0.0, causal)
        assert np.max(np.abs(dq)) == 0.0 and np.max(np.abs(dk)) == 0.0, "scale 0: dQ, dK must be 0"
        want = np.zeros(dv.shape)
        for i in range(7):
            vis = min(9, i + 1) if causal else 9
            want[:, :, :vis] += do[:, :, i:i + 1].astype(np.float64) / vis
        _close(dv, want, 1e-13, f"scale 0: dV (causal={causal})")


def pin_invariants(lib):
    B, H, Nq, Nk, d = 2, 2, 9, 12, 6
    # dyadic values: the shifted keys below are exact in float32
    q, k, v, do = _case(41, B, H, Nq, Nk, d, grid=24)
    scale = 0.4
    for causal in (False, True):
        dq, dk, dv = _bwd(lib, q, k, v, do, scale, causal)
        assert np.max(np.abs(dk.sum(axis=2))) < 1e-12 * max(1.0, np.max(np.abs(dk))), \
            f"sum_j dK_j must be 0 (causal={causal})"
        # queries that see no key do not exist (every row sees key 0)
        _close(dv.sum(axis=2), do.astype(np.float64).sum(axis=2), 1e-12,
               f"sum_j dV_j = sum_i dO_i (causal={causal})")
        # key shift: the same u added to every key leaves dQ
        u = _rng(42).integers(-4, 5, size=d).astype(np.float32) / np.float32(4)
        dq2, _, _ = _bwd(lib, q, k + u, v, do, scale, causal)
        _close(dq2, dq, 1e-11, f"dQ under a common key shift (causal={causal})")
        # sampled rows agree with the full result
        qr = np.array([0, 3, 8], dtype=np.int32)
        kr = np.array([11, 0, 5], dtype=np.int32)
        sq, sk, sv = _bwd(lib, q, k, v, do, scale, causal, qrows=qr, krows=kr)
        _close(sq, dq[:, :, qr], 1e-14, "sampled dQ rows")
        _close(sk, dk[:, :, kr], 1e-14, "sampled dK rows")
        _close(sv, dv[:, :, kr], 1e-14, "sampled dV rows")
    # permutation of keys and values together (non-causal)
    perm = _rng(43).permutation(Nk)
    dq, dk, dv = _bwd(lib, q, k, v, do, scale, False)
    pq, pk, pv = _bwd(lib, q, k[:, :, perm], v[:, :, perm], do, scale, False)
    _close(pq, dq, 1e-12, "dQ under a key permutation")
    _close(pk, dk[:, :, perm], 1e-12, "dK under a key permutation")
    _close(pv, dv[:, :, perm], 1e-12, "dV under a key permutation")


ALL_BWD_PINS = [
    pin_torch_autograd,
    pin_finite_differences,
    pin_closed_forms,
    pin_invariants,
]

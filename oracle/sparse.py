"""Block-sparse attention for the oracle -- TEST INFRASTRUCTURE ONLY.

[nanhubrain] "SparseFlashAttention": the forward pass with a sparse mask
over (query block, key block) pairs; the key blocks the mask marks as not
needed are skipped.  Written here as its plain definition: key j is visible
to query i iff block_mask[i // bq, j // bk] is nonzero (and j <= i when
causal); softmax attention over the visible keys in float64 (numpy), one
head at a time, with the row max subtracted.  A row with no visible key
gives O = 0 and LSE = -inf.  ``attn_bwd_block_sparse`` gives the gradients
of the same attention by their plain definition.
"""
from __future__ import annotations

import numpy as np


def attn_fwd_block_sparse(q, k, v, block_mask, *, bq: int, bk: int, scale: float, causal: bool = False,
                          rows=None):
    """O [R, d] and LSE [R] (float64) of one head.

    q [Nq, d], k and v [Nk, d] (float values), block_mask [ceil(Nq/bq),
    ceil(Nk/bk)] (nonzero = the block is computed); ``rows``: optional query
    indices (default all)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    Nq, Nk = q.shape[0], k.shape[0]
    rows = np.arange(Nq) if rows is None else np.asarray(rows)
    cols = np.arange(Nk)
    o = np.zeros((len(rows), q.shape[1]))
    lse = np.full(len(rows), -np.inf)
    for n, i in enumerate(rows):
        vis = block_mask[i // bq, cols // bk] != 0
        if causal:
            vis &= cols <= i
        if not vis.any():
            continue
        s = scale * (k[vis] @ q[i])
        m = s.max()
        p = np.exp(s - m)
        o[n] = (p @ v[vis]) / p.sum()
        lse[n] = m + np.log(p.sum())
    return o, lse


def attn_bwd_block_sparse(q, k, v, do, block_mask, *, bq: int, bk: int, scale: float, causal: bool = False,
                          qrows=None, krows=None, chunk: int = 512):
    """Gradients (dQ [RQ, d], dK [RK, d], dV [RK, d]) (float64) of one head of
    ``attn_fwd_block_sparse`` for an upstream gradient dO [Nq, d].

    The plain definition over each row's visible keys ([nanhubrain]
    "backward recomputation", with the row term over the whole visible row):
    P_ij = exp(scale q_i.k_j - LSE_i), dP_ij = dO_i.v_j,
    D_i = sum_j P_ij dP_ij, dS_ij = P_ij (dP_ij - D_i),
    dQ_i = scale sum_j dS_ij k_j, dK_j = scale sum_i dS_ij q_i,
    dV_j = sum_i P_ij dO_i.  A row with no visible key has no gradient and
    passes none on.  ``qrows`` / ``krows``: optional row / key indices
    (default all).  The row statistics are computed ``chunk`` rows at a time.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    Nq, Nk = q.shape[0], k.shape[0]
    qrows = np.arange(Nq) if qrows is None else np.asarray(qrows)
    krows = np.arange(Nk) if krows is None else np.asarray(krows)
    cols = np.arange(Nk)

    def visible(rows):
        vis = block_mask[rows[:, None] // bq, cols[None, :] // bk] != 0
        if causal:
            vis &= cols[None, :] <= rows[:, None]
        return vis

    # row statistics of every query: LSE_i and D_i over the visible keys
    lse = np.full(Nq, -np.inf)
    D = np.zeros(Nq)
    for r0 in range(0, Nq, chunk):
        rows = np.arange(r0, min(Nq, r0 + chunk))
        vis = visible(rows)
        s = np.where(vis, scale * (q[rows] @ k.T), -np.inf)
        top = s.max(axis=1)
        live = vis.any(axis=1)
        top_safe = np.where(live, top, 0.0)
        p = np.where(vis, np.exp(s - top_safe[:, None]), 0.0)
        z = p.sum(axis=1)
        lse[rows] = np.where(live, top_safe + np.log(np.where(live, z, 1.0)), -np.inf)
        p = p / np.where(live, z, 1.0)[:, None]
        D[rows] = np.sum(p * (do[rows] @ v.T), axis=1)

    def probs(rows, cs, vis):
        s = scale * (q[rows] @ k[cs].T)
        lse_r = np.where(np.isfinite(lse[rows]), lse[rows], 0.0)
        return np.where(vis, np.exp(np.where(vis, s - lse_r[:, None], 0.0)), 0.0)

    # dQ of the requested rows
    vis = visible(qrows)
    p = probs(qrows, cols, vis)
    ds = p * ((do[qrows] @ v.T) - D[qrows][:, None])
    dq = scale * (ds @ k)
    # dK, dV of the requested keys, over every query
    allq = np.arange(Nq)
    dk = np.zeros((len(krows), q.shape[1]))
    dv = np.zeros((len(krows), q.shape[1]))
    for r0 in range(0, Nq, chunk):
        rows = allq[r0:r0 + chunk]
        vis = block_mask[rows[:, None] // bq, krows[None, :] // bk] != 0
        if causal:
            vis &= krows[None, :] <= rows[:, None]
        p = probs(rows, krows, vis)
        ds = p * ((do[rows] @ v[krows].T) - D[rows][:, None])
        dk += scale * (ds.T @ q[rows])
        dv += p.T @ do[rows]
    return dq, dk, dv

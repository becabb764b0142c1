"""Block-sparse attention for the oracle -- TEST INFRASTRUCTURE ONLY.

[nanhubrain] "SparseFlashAttention": the forward pass with a sparse mask
over (query block, key block) pairs; the key blocks the mask marks as not
needed are skipped.  Written here as its plain definition: key j is visible
to query i iff block_mask[i // bq, j // bk] is nonzero (and j <= i when
causal); softmax attention over the visible keys in float64 (numpy), one
head at a time, with the row max subtracted.  A row with no visible key
gives O = 0 and LSE = -inf.
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

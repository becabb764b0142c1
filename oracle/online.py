"""The pages' own algorithm in fp64: tiled forward with the online softmax.

TEST INFRASTRUCTURE ONLY (see the package docstring).  This is the method as
the pages describe it -- outer loop over query blocks, inner loop over key/value
blocks, running statistics (row max m, row sum l) merged block by block, and a
rescaled output accumulator -- written in numpy float64 so that the tests can
check that the recurrence over *any* block split reaches the two-pass
definition in ``oracle.c``.

Sources:
* [nanhubrain] section "tiling skeleton": the Q-block-outer / KV-block-inner
  loop, the per-block max m_ij, exponentials P_ij = exp(S_ij - m_ij) and sum
  l_ij, then the merge with the previous statistics through the two rescale
  factors exp(m_prev - m_new) and exp(m_ij - m_new); after the inner loop the
  accumulator is divided by the row sum once and written with the statistics.
* [nanhubrain] section "online softmax mathematics": the single-vector step
  (m_cur = max(m_prev, m_t); l_cur = l_prev e^(m_prev-m_cur) + s_t e^(m_t-m_cur))
  and the argument that the rescale is exact, so any split gives the global
  softmax.
* [ascendai] section 2.2: the same merge written against the new maximum
  directly (exp(S - new_max) for the current block, one correction factor for
  the previous accumulator and sum).

Reading taken where the pages are inconsistent: the tiling-skeleton listing
divides the current block's probabilities by l_ij inside the accumulator
update and then divides by the row sum again after the loop; that normalises
twice and is wrong even for a single block.  Here the accumulator stays
unnormalised (o = o * rescale_prev + rescale_cur * (P_ij @ v_j)) and is divided
by the row sum exactly once at the end, which is what [ascendai] section 2.2
and the exactness argument require.  The [pwwt] "online softmax update" that
divides by the new sum at every step is likewise not used.

Rows whose every key in a block is masked (causal) have m_ij = -inf; their
block contributes nothing (rescale_cur = 0, P_ij = 0).  A row with no visible
key so far keeps m = -inf and rescale_prev = 0.
"""
from __future__ import annotations

import numpy as np


def _blocks(n: int, splits):
    """Block boundaries [(a, b), ...] covering [0, n).  ``splits`` is either a
    block size (int) or a sorted list of interior cut points."""
    if isinstance(splits, (int, np.integer)):
        size = int(splits)
        if size < 1:
            raise ValueError("block size must be >= 1")
        cuts = list(range(size, n, size))
    else:
        cuts = [int(c) for c in splits if 0 < int(c) < n]
        if cuts != sorted(set(cuts)):
            raise ValueError("cut points must be strictly increasing")
    edges = [0] + cuts + [n]
    return list(zip(edges[:-1], edges[1:]))


def online_softmax_stats(x, splits):
    """Running (m, l) over a 1-D vector processed block by block
    ([nanhubrain] "online softmax mathematics")."""
    x = np.asarray(x, dtype=np.float64)
    m_prev, l_prev = -np.inf, 0.0
    for a, b in _blocks(x.size, splits):
        x_t = x[a:b]
        m_t = x_t.max()
        s_t = np.exp(x_t - m_t).sum()
        m_cur = max(m_prev, m_t)
        l_cur = (l_prev * np.exp(m_prev - m_cur) if np.isfinite(m_prev) else 0.0) \
            + s_t * np.exp(m_t - m_cur)
        m_prev, l_prev = m_cur, l_cur
    return m_prev, l_prev


def _head_online(q, k, v, scale, causal, q_splits, kv_splits, form):
    Nq, d = q.shape
    Nk = k.shape[0]
    O = np.zeros((Nq, d))
    row_max = np.full((Nq,), -np.inf)
    row_sum = np.zeros((Nq,))
    for i0, i1 in _blocks(Nq, q_splits):
        q_i = q[i0:i1]
        m_prev = np.full((i1 - i0, 1), -np.inf)
        l_prev = np.zeros((i1 - i0, 1))
        o_i = np.zeros((i1 - i0, d))
        for j0, j1 in _blocks(Nk, kv_splits):
            k_j, v_j = k[j0:j1], v[j0:j1]
            S = scale * (q_i @ k_j.T)
            if causal:
                qi_idx = np.arange(i0, i1)[:, None]
                kj_idx = np.arange(j0, j1)[None, :]
                S = np.where(kj_idx > qi_idx, -np.inf, S)
            m_ij = S.max(axis=1, keepdims=True)
            live = np.isfinite(m_ij)
            m_new = np.maximum(m_prev, m_ij)
            prev_live = np.isfinite(m_prev)
            if form == "block_max":
                # [nanhubrain] tiling skeleton: exponentials against the block max,
                # then both sides rescaled to the new max.
                P = np.where(live, np.exp(S - np.where(live, m_ij, 0.0)), 0.0)
                l_ij = P.sum(axis=1, keepdims=True)
                rescale_prev = np.where(prev_live, np.exp(np.where(prev_live, m_prev - m_new, 0.0)), 0.0)
                rescale_cur = np.where(live, np.exp(np.where(live, m_ij - m_new, 0.0)), 0.0)
                o_i = o_i * rescale_prev + rescale_cur * (P @ v_j)
                l_prev = l_prev * rescale_prev + l_ij * rescale_cur
            elif form == "new_max":
                # [ascendai] 2.2: exponentials against the new max directly.
                new_live = np.isfinite(m_new)
                base = np.where(new_live, m_new, 0.0)
                P = np.where(new_live, np.exp(S - base), 0.0)
                correction = np.where(prev_live, np.exp(np.where(prev_live, m_prev - m_new, 0.0)), 0.0)
                l_prev = l_prev * correction + P.sum(axis=1, keepdims=True)
                o_i = o_i * correction + P @ v_j
            else:
                raise ValueError(f"unknown form {form!r}")
            m_prev = m_new
        O[i0:i1] = o_i / l_prev
        row_max[i0:i1] = m_prev[:, 0]
        row_sum[i0:i1] = l_prev[:, 0]
    return O, row_max, row_sum


def attn_fwd_online(q, k, v, *, scale: float, causal: bool = False,
                    layout: str = "BHND", q_splits=128, kv_splits=128,
                    form: str = "block_max"):
    """O [B,H,Nq,d], LSE [B,H,Nq], row_max, row_sum (all float64) by the tiled
    online-softmax recurrence.  q, k, v as for ``oracle.attn_fwd``."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if layout == "BSND":
        q = q.transpose(0, 2, 1, 3)
        k = k.transpose(0, 2, 1, 3)
        v = v.transpose(0, 2, 1, 3)
    elif layout != "BHND":
        raise ValueError(f"unknown layout {layout!r}")
    B, H, Nq, d = q.shape
    O = np.empty((B, H, Nq, d))
    M = np.empty((B, H, Nq))
    L = np.empty((B, H, Nq))
    for b in range(B):
        for h in range(H):
            O[b, h], M[b, h], L[b, h] = _head_online(
                q[b, h], k[b, h], v[b, h], scale, causal, q_splits, kv_splits, form)
    lse = M + np.log(L)
    return O, lse, M, L

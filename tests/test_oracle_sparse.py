"""Pins of the block-sparse oracle (oracle/sparse.py): torch's CPU
scaled_dot_product_attention in float64 with the expanded boolean mask
(library routine); an all-ones mask equals the plain oracle; an all-zero
mask row gives O = 0, LSE = -inf; a single active block of identical keys
gives the mean of its values; permuting key blocks together with the mask's
columns changes nothing (non-causal)."""
import numpy as np

import oracle
from oracle import sparse


def _rng(s):
    return np.random.Generator(np.random.PCG64(s))


def _case(seed, Nq, Nk, d, nqb, nkb, density=0.5):
    g = _rng(seed)
    q = g.standard_normal((Nq, d)).astype(np.float32)
    k = g.standard_normal((Nk, d)).astype(np.float32)
    v = g.standard_normal((Nk, d)).astype(np.float32)
    mask = (g.random((nqb, nkb)) < density).astype(np.uint8)
    return q, k, v, mask


def test_torch_masked_sdpa():
    import torch
    import torch.nn.functional as F
    for seed, causal in ((1, False), (2, True)):
        q, k, v, mask = _case(seed, 37, 45, 6, 5, 6)
        o, lse = sparse.attn_fwd_block_sparse(q, k, v, mask, bq=8, bk=8, scale=0.4, causal=causal)
        full = mask[np.arange(37)[:, None] // 8, np.arange(45)[None, :] // 8] != 0
        if causal:
            full &= np.arange(45)[None, :] <= np.arange(37)[:, None]
        live = full.any(axis=1)
        tq, tk, tv = (torch.tensor(x, dtype=torch.float64) for x in (q, k, v))
        want = F.scaled_dot_product_attention(tq[None], tk[None], tv[None], attn_mask=torch.tensor(full)[None],
                                              scale=0.4)[0].numpy()
        s = 0.4 * (tq @ tk.T)
        want_lse = torch.logsumexp(s.masked_fill(~torch.tensor(full), float("-inf")), dim=-1).numpy()
        assert np.max(np.abs(o[live] - want[live])) < 1e-12
        assert np.max(np.abs(lse[live] - want_lse[live])) < 1e-12
        assert np.all(o[~live] == 0) and np.all(np.isneginf(lse[~live]))


def test_all_ones_is_plain():
    q, k, v, _ = _case(3, 30, 50, 4, 4, 7)
    ones = np.ones((4, 7), dtype=np.uint8)
    for causal in (False, True):
        o, lse = sparse.attn_fwd_block_sparse(q, k, v, ones, bq=8, bk=8, scale=0.5, causal=causal)
        o2, lse2 = oracle.attn_fwd(q[None, None], k[None, None], v[None, None], scale=0.5, causal=causal)
        assert np.max(np.abs(o - o2[0, 0])) < 1e-13 and np.max(np.abs(lse - lse2[0, 0])) < 1e-13


def test_closed_forms():
    q, k, v, _ = _case(4, 16, 32, 4, 2, 4)
    mask = np.zeros((2, 4), dtype=np.uint8)
    mask[0, 2] = 1                                     # query block 0 sees key block 2 only
    k[16:24] = k[16]                                   # identical keys in that block
    o, lse = sparse.attn_fwd_block_sparse(q, k, v, mask, bq=8, bk=8, scale=0.7)
    want = v[16:24].astype(np.float64).mean(axis=0)
    assert np.max(np.abs(o[:8] - want)) < 1e-13
    assert np.allclose(lse[:8], 0.7 * (q[:8].astype(np.float64) @ k[16].astype(np.float64)) + np.log(8), atol=1e-12)
    assert np.all(o[8:] == 0) and np.all(np.isneginf(lse[8:]))   # query block 1 sees nothing


def test_block_permutation():
    q, k, v, mask = _case(5, 24, 40, 5, 3, 5)
    perm = _rng(6).permutation(5)
    idx = np.concatenate([np.arange(8 * b, 8 * b + 8) for b in perm])
    o, lse = sparse.attn_fwd_block_sparse(q, k, v, mask, bq=8, bk=8, scale=0.3)
    o2, lse2 = sparse.attn_fwd_block_sparse(q, k[idx], v[idx], mask[:, perm], bq=8, bk=8, scale=0.3)
    assert np.max(np.abs(o - o2)) < 1e-13 and np.max(np.abs(lse - lse2)[np.isfinite(lse)]) < 1e-13

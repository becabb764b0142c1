"""Pins of the block-sparse backward oracle (oracle/sparse.py,
attn_bwd_block_sparse): torch's autograd through its CPU
scaled_dot_product_attention in float64 with the expanded boolean mask
(library routine); an all-ones mask equals the pinned plain backward
oracle; a query block with no active key block has zero dQ and adds nothing
to dK or dV; a key block no query sees gets zero dK and dV; the sampled-row
mode equals the full result."""
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
    do = g.standard_normal((Nq, d)).astype(np.float32)
    mask = (g.random((nqb, nkb)) < density).astype(np.uint8)
    return q, k, v, do, mask


def _full_mask(mask, Nq, Nk, bq, bk, causal):
    full = mask[np.arange(Nq)[:, None] // bq, np.arange(Nk)[None, :] // bk] != 0
    if causal:
        full &= np.arange(Nk)[None, :] <= np.arange(Nq)[:, None]
    return full


def test_torch_autograd():
    import torch
    import torch.nn.functional as F
    for seed, causal in ((11, False), (12, True)):
        q, k, v, do, mask = _case(seed, 40, 48, 6, 5, 6, density=0.6)
        mask[:, 0] = 1                                   # every row sees a key (torch gives NaN otherwise)
        full = _full_mask(mask, 40, 48, 8, 8, causal)
        assert full.any(axis=1).all()
        dq, dk, dv = sparse.attn_bwd_block_sparse(q, k, v, do, mask, bq=8, bk=8, scale=0.35, causal=causal)
        tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
        o = F.scaled_dot_product_attention(tq[None], tk[None], tv[None], attn_mask=torch.tensor(full)[None], scale=0.35)
        o.backward(torch.tensor(do, dtype=torch.float64)[None])
        for name, got, t in (("dQ", dq, tq), ("dK", dk, tk), ("dV", dv, tv)):
            err = float(np.max(np.abs(got - t.grad.numpy())))
            assert err < 1e-11, f"{name} vs torch autograd: {err:.2e}"


def test_all_ones_is_plain():
    q, k, v, do, _ = _case(13, 33, 41, 5, 5, 6)
    ones = np.ones((5, 6), dtype=np.uint8)
    for causal in (False, True):
        a = sparse.attn_bwd_block_sparse(q, k, v, do, ones, bq=8, bk=8, scale=0.5, causal=causal)
        b = oracle.attn_bwd(q[None, None], k[None, None], v[None, None], do[None, None], scale=0.5, causal=causal)
        for x, y in zip(a, b):
            assert np.max(np.abs(x - y[0, 0])) < 1e-12


def test_empty_blocks():
    q, k, v, do, mask = _case(14, 32, 32, 4, 4, 4, density=0.7)
    mask[1, :] = 0                                       # query block 1 sees nothing
    mask[:, 2] = 0                                       # key block 2 is seen by no query
    dq, dk, dv = sparse.attn_bwd_block_sparse(q, k, v, do, mask, bq=8, bk=8, scale=0.6)
    assert np.all(dq[8:16] == 0.0), "rows without keys: dQ = 0"
    assert np.all(dk[16:24] == 0.0) and np.all(dv[16:24] == 0.0), "keys no query sees: dK = dV = 0"
    do2 = do.copy()
    do2[8:16] *= 5.0                                     # the empty rows' upstream gradient
    _, dk2, dv2 = sparse.attn_bwd_block_sparse(q, k, v, do2, mask, bq=8, bk=8, scale=0.6)
    assert np.array_equal(dk, dk2) and np.array_equal(dv, dv2), "rows without keys pass nothing on"


def test_sampled_rows_equal_full():
    q, k, v, do, mask = _case(15, 50, 60, 4, 7, 8)
    full = sparse.attn_bwd_block_sparse(q, k, v, do, mask, bq=8, bk=8, scale=0.45, causal=True, chunk=16)
    qr, kr = np.array([49, 0, 13]), np.array([59, 7, 30, 31])
    sub = sparse.attn_bwd_block_sparse(q, k, v, do, mask, bq=8, bk=8, scale=0.45, causal=True, qrows=qr,
                                       krows=kr, chunk=16)
    assert np.max(np.abs(sub[0] - full[0][qr])) < 1e-13
    assert np.max(np.abs(sub[1] - full[1][kr])) < 1e-13 and np.max(np.abs(sub[2] - full[2][kr])) < 1e-13

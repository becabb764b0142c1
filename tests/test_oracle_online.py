"""The pages' online-softmax recurrence (oracle/online.py) over arbitrary block
splits reaches the two-pass definition (oracle.c): the exactness argument of
[nanhubrain] "online softmax mathematics"."""
import math

import numpy as np
import pytest

from oracle import online


def _case(seed, B, H, Nq, Nk, d, sigma=1.0):
    g = np.random.Generator(np.random.PCG64(seed))
    return tuple((g.standard_normal(s) * sg).astype(np.float32)
                 for s, sg in (((B, H, Nq, d), sigma), ((B, H, Nk, d), sigma), ((B, H, Nk, d), 1.0)))


SPLITS = [1, 3, 16, 64, [5], [1, 2, 3, 10], [7, 8, 20, 21]]


@pytest.mark.parametrize("form", ["block_max", "new_max"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("qs,ks", [(1, 1), (16, 3), ([5], [1, 2, 3, 10]), (7, [7, 8, 20, 21]), (64, 64)])
def test_online_equals_two_pass(oracle_lib, form, causal, qs, ks):
    q, k, v = _case(11, 1, 2, 23, 29, 8, sigma=2.0)
    o2, l2 = oracle_lib.attn_fwd(q, k, v, scale=0.5, causal=causal)
    o1, l1, m, l = online.attn_fwd_online(q, k, v, scale=0.5, causal=causal,
                                          q_splits=qs, kv_splits=ks, form=form)
    assert np.abs(o1 - o2).max() < 1e-13
    assert np.abs(l1 - l2).max() < 1e-13
    assert np.all(l >= 1.0 - 1e-15)          # the max key contributes exp(0) = 1


def test_online_bsnd_and_peaked(oracle_lib):
    q, k, v = _case(12, 2, 3, 40, 33, 16)
    k[:, :, 5] *= 8
    k[:, :, 30] *= 8
    qb, kb, vb = (np.ascontiguousarray(x.transpose(0, 2, 1, 3)) for x in (q, k, v))
    o2, l2 = oracle_lib.attn_fwd(qb, kb, vb, scale=0.25, causal=True, layout="BSND")
    o1, l1, _, _ = online.attn_fwd_online(qb, kb, vb, scale=0.25, causal=True, layout="BSND",
                                          q_splits=8, kv_splits=[4, 5, 6, 31])
    assert np.abs(o1 - o2).max() < 1e-13 and np.abs(l1 - l2).max() < 1e-13


@pytest.mark.parametrize("splits", SPLITS)
def test_online_stats_match_definition(splits):
    x = np.random.Generator(np.random.PCG64(13)).standard_normal(97) * 20
    m, l = online.online_softmax_stats(x, splits)
    assert m == x.max()
    assert abs(l - math.fsum(math.exp(t - x.max()) for t in x)) < 1e-12 * l


def test_online_page_listing_double_normalisation_is_wrong(oracle_lib):
    """The reading taken for the tiling-skeleton listing: dividing the block's
    probabilities by l_ij inside the update *and* by the row sum at the end
    does not give softmax attention even for one block -- so that listing is
    not followed literally."""
    q, k, v = _case(14, 1, 1, 4, 6, 4)
    o_ref, _ = oracle_lib.attn_fwd(q, k, v, scale=0.5)
    s = 0.5 * q[0, 0].astype(np.float64) @ k[0, 0].astype(np.float64).T
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    l = p.sum(axis=1, keepdims=True)
    literal = ((p / l) @ v[0, 0].astype(np.float64)) / l   # one block, as printed
    assert np.abs(literal - o_ref[0, 0]).max() > 1e-3


def test_blocks_cover_range():
    assert online._blocks(10, 3) == [(0, 3), (3, 6), (6, 9), (9, 10)]
    assert online._blocks(10, [2, 7]) == [(0, 2), (2, 7), (7, 10)]
    with pytest.raises(ValueError):
        online._blocks(10, [7, 2])

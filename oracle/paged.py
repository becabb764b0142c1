"""Paged KV cache gather for the decode oracle -- TEST INFRASTRUCTURE ONLY.

[nanhubrain] "GatherPAKVCache": the cache is stored in blocks; for a sequence
of length seq_len, logical block i (i < ceil(seq_len / block_size)) lives in
physical block block_tables[i]; the blocks are read in logical order and
concatenated along the token axis, and in GQA mode only the KV heads listed
in head_indices are kept.  Here the cache is [num_blocks, block_size, heads,
d] and the result is cut to seq_len tokens.  Pure data movement in numpy; no
arithmetic of the attention method.
"""
from __future__ import annotations

import numpy as np


def gather_paged_kv(key_cache, value_cache, block_table, seq_len, head_indices=None):
    """(K, V) [seq_len, heads, d] of one sequence from the paged cache."""
    block_size = key_cache.shape[1]
    n_blocks = (int(seq_len) + block_size - 1) // block_size
    ks, vs = [], []
    for i in range(n_blocks):
        phys = int(block_table[i])                # logical block -> physical block
        kb, vb = key_cache[phys], value_cache[phys]
        if head_indices is not None:
            kb, vb = kb[:, head_indices, :], vb[:, head_indices, :]
        ks.append(kb)
        vs.append(vb)
    k = np.concatenate(ks, axis=0)[:seq_len]
    v = np.concatenate(vs, axis=0)[:seq_len]
    return k, v


def decode_reference(lib, q, key_cache, value_cache, block_tables, seq_lens, *, scale, causal):
    """O [B, Nq, H, d] and LSE [B, H, Nq] (float64) of decode attention: the
    Nq new tokens of sequence b sit at positions L_b - Nq .. L_b - 1 and
    attend to the gathered keys 0 .. L_b - 1 (causal: token t to keys
    j <= L_b - Nq + t, i.e. the band's right edge L_b - Nq), grouped KV heads
    as in ``lib.attn_fwd_ex``."""
    B, Nq, H, d = q.shape
    o = np.zeros((B, Nq, H, d))
    lse = np.full((B, H, Nq), -np.inf)
    for b in range(B):
        L = int(seq_lens[b])
        if causal and L < Nq:
            raise ValueError("causal decode needs every sequence to hold its Nq new tokens")
        if L == 0:
            continue
        k, v = gather_paged_kv(key_cache, value_cache, block_tables[b], L)
        window = (-1, L - Nq) if causal else (-1, -1)
        ob, lb = lib.attn_fwd_ex(q[b:b + 1], k[None], v[None], scale=scale, causal=False, window=window,
                                 layout="BSND")
        o[b] = ob[0].transpose(1, 0, 2)
        lse[b] = lb[0]
    return o, lse

"""Seeded synthetic inputs for the attention forward workloads.

This module is the only code shared by the GPU path's tests and the CPU oracle:
it draws random numbers and rounds them to the storage dtype, and holds none of
the attention arithmetic.

Recipe (one ``numpy.random.Generator(PCG64(seed))`` per tensor, seed =
1000 * config_id + t with t = 0 for Q, 1 for K, 2 for V, 3 for the choice of
peaked key rows, 4 for the upstream gradient dO of the backward pass):

* values are float32 ``standard_normal`` draws in the *storage order* of the
  workload's layout (BHND = [B,H,N,d], BSND = [B,N,H,d]), times the tensor's
  standard deviation;
* in the long-context workload, round(1% of Nk) distinct key positions per
  (b, h) are drawn and those K rows multiplied by 8 (exact in binary floating
  point, so the order against rounding does not matter);
* bf16 workloads then round every value to bf16, round-to-nearest-even.  The
  GPU receives the bf16 bits; the oracle receives the same values widened to
  float32 (exact).

The shapes are those of the pages' workloads: an LLaMA-13B-like prefill
(32 heads of 128, [pwwt] "measured performance"), the B=4 H=32 D=128
self-attention of [ascendai] section 4.3, a Stable-Diffusion-style
cross-attention ([ascendai] section 4.2: 128x128 latent tokens against a
77-token context), and a 128K causal context ([ascendai] sections 1.3 and 4.3).
Trained weights do not exist here: N(0, sigma^2) activations of those shapes
stand in for the models' activations.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    cid: int            # config id, used in the seeds
    name: str
    B: int
    H: int
    Nq: int
    Nk: int
    d: int
    dtype: str          # "bf16" or "f32"
    layout: str         # "BHND" or "BSND"
    causal: bool
    sigma_q: float = 1.0
    sigma_k: float = 1.0
    sigma_v: float = 1.0
    peaked_frac: float = 0.0   # fraction of K rows scaled by peaked_mult
    peaked_mult: float = 8.0
    Hkv: int = 0               # key/value heads (0: H); query head h reads KV head h // (H // Hkv)
    window: tuple = (-1, -1)   # band (left, right): keys i-left .. i+right visible; negative: unbounded
    block_sparse: bool = False  # a block mask from make_block_mask decides which key blocks are computed

    @property
    def kv_heads(self) -> int:
        return self.Hkv or self.H

    @property
    def visible_pairs(self) -> int:
        """Visible (query, key) pairs of one head under the causal flag and the band."""
        lo_w, hi_w = self.window
        total = 0
        for i in range(self.Nq):
            lo = max(0, i - lo_w) if lo_w >= 0 else 0
            hi = min(self.Nk - 1, i + hi_w) if hi_w >= 0 else self.Nk - 1
            if self.causal:
                hi = min(hi, i)
            total += max(0, hi - lo + 1)
        return total

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def flops(self) -> float:
        """4*B*H*Nq*Nk*d, halved for causal (the dense count, not N(N+1)/2);
        with a band, 4*B*H*d per visible (query, key) pair."""
        if self.window != (-1, -1):
            return 4.0 * self.B * self.H * self.d * self.visible_pairs
        f = 4.0 * self.B * self.H * self.Nq * self.Nk * self.d
        return f / 2 if self.causal else f

    def q_shape(self):
        return self._shape(self.Nq)

    def kv_shape(self):
        return self._shape(self.Nk, self.kv_heads)

    def _shape(self, n, heads=None):
        heads = self.H if heads is None else heads
        if self.layout == "BHND":
            return (self.B, heads, n, self.d)
        return (self.B, n, heads, self.d)

    def scaled(self, **changes) -> "Workload":
        return dataclasses.replace(self, **changes)


WORKLOADS = {
    "tiny_f32": Workload(1, "tiny_f32", 1, 2, 256, 256, 64, "f32", "BHND", False),
    "llama_prefill_causal": Workload(2, "llama_prefill_causal", 1, 32, 4096, 4096, 128,
                                     "bf16", "BSND", True),
    "selfattn_b4h32n8k": Workload(3, "selfattn_b4h32n8k", 4, 32, 8192, 8192, 128,
                                  "bf16", "BHND", False),
    "sd_crossattn": Workload(4, "sd_crossattn", 2, 8, 16384, 77, 64, "bf16", "BHND", False,
                             sigma_k=0.5, sigma_v=0.5),
    "long_causal_128k": Workload(5, "long_causal_128k", 1, 32, 131072, 131072, 128,
                                 "bf16", "BSND", True, peaked_frac=0.01),
    # the inference-side variants of the pages' next rows: grouped KV heads
    # ([nanhubrain] "GatherPAKVCache", GQA/MQA) under a causal sliding window
    # ([pwwt] pre_tokens / next_tokens), at the LLaMA-like 32 x 128 head shape
    "gqa_swa_prefill": Workload(6, "gqa_swa_prefill", 1, 32, 16384, 16384, 128, "bf16", "BSND", True,
                                Hkv=8, window=(4095, -1)),
    # block-sparse attention of the BigBird kind ([nanhubrain] "SparseFlashAttention"):
    # local, global and random key blocks per query block
    "sparse_bigbird": Workload(8, "sparse_bigbird", 2, 16, 16384, 16384, 128, "bf16", "BHND", False,
                               block_sparse=True),
}

# granularity of block masks: queries x keys per block
SPARSE_BQ, SPARSE_BK = 256, 64


def make_block_mask(w: Workload, seed_base: int | None = None, n_random: int = 8) -> np.ndarray:
    """uint8 [B, H, ceil(Nq/256), ceil(Nk/64)]: for each (b, h) and query block
    qb, the key blocks overlapping keys [256*qb - 256, 256*qb + 512) (local),
    the first 4 key blocks (global) and n_random key blocks drawn from seed
    1000*cid+7 (random), the BigBird pattern."""
    base = 1000 * w.cid if seed_base is None else seed_base
    nqb = (w.Nq + SPARSE_BQ - 1) // SPARSE_BQ
    nkb = (w.Nk + SPARSE_BK - 1) // SPARSE_BK
    g = np.random.Generator(np.random.PCG64(base + 7))
    mask = np.zeros((w.B, w.H, nqb, nkb), dtype=np.uint8)
    for qb in range(nqb):
        lo = max(0, (SPARSE_BQ * qb - SPARSE_BQ) // SPARSE_BK)
        hi = min(nkb, (SPARSE_BQ * qb + 2 * SPARSE_BQ + SPARSE_BK - 1) // SPARSE_BK)
        mask[:, :, qb, lo:hi] = 1
        mask[:, :, qb, :min(4, nkb)] = 1
    rnd = g.integers(0, nkb, size=(w.B, w.H, nqb, n_random))
    for b in range(w.B):
        for h in range(w.H):
            for qb in range(nqb):
                mask[b, h, qb, rnd[b, h, qb]] = 1
    return mask
BY_ID = {w.cid: w for w in WORKLOADS.values()}


# ----------------------------------------------------------------------------
# bf16 storage conversion (round to nearest, ties to even)

_CHUNK = 1 << 24


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) of float32 values, round-to-nearest-even.
    Inputs here are finite; NaN handling is not needed."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    flat = x.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint16)
    for a in range(0, flat.size, _CHUNK):
        u = flat[a:a + _CHUNK].view(np.uint32)
        bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
        out[a:a + _CHUNK] = ((u + bias) >> np.uint32(16)).astype(np.uint16)
    return out.reshape(x.shape)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    flat = b.reshape(-1)
    out = np.empty(flat.shape, dtype=np.float32)
    ov = out.view(np.uint32)
    for a in range(0, flat.size, _CHUNK):
        ov[a:a + _CHUNK] = flat[a:a + _CHUNK].astype(np.uint32) << np.uint32(16)
    return out.reshape(b.shape)


# ----------------------------------------------------------------------------

@dataclasses.dataclass
class Inputs:
    w: Workload
    q: np.ndarray                 # float32 values (exact input values), storage order
    k: np.ndarray
    v: np.ndarray
    q_bits: np.ndarray | None     # uint16 bf16 bits (bf16 workloads only)
    k_bits: np.ndarray | None
    v_bits: np.ndarray | None
    peaked: np.ndarray | None     # [B, H, n_peaked] key positions scaled up, or None


def _draw(seed: int, shape, sigma: float) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(seed))
    x = g.standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return x


def peaked_positions(w: Workload, seed_base: int | None = None) -> np.ndarray | None:
    """Key positions whose K rows are scaled, per (b, h), drawn from seed
    1000*cid+3 (or seed_base+3)."""
    if w.peaked_frac <= 0:
        return None
    base = 1000 * w.cid if seed_base is None else seed_base
    n = int(round(w.peaked_frac * w.Nk))
    g = np.random.Generator(np.random.PCG64(base + 3))
    pos = np.empty((w.B, w.kv_heads, n), dtype=np.int64)
    for b in range(w.B):
        for h in range(w.kv_heads):
            pos[b, h] = np.sort(g.choice(w.Nk, size=n, replace=False))
    return pos


def make_inputs(w: Workload, seed_base: int | None = None) -> Inputs:
    """Inputs of workload ``w``.  ``seed_base`` replaces 1000*cid (for extra
    cases of the same recipe at other shapes)."""
    base = 1000 * w.cid if seed_base is None else seed_base
    q = _draw(base + 0, w.q_shape(), w.sigma_q)
    k = _draw(base + 1, w.kv_shape(), w.sigma_k)
    v = _draw(base + 2, w.kv_shape(), w.sigma_v)
    pos = peaked_positions(w, seed_base)
    if pos is not None:
        mult = np.float32(w.peaked_mult)
        for b in range(w.B):
            for h in range(w.kv_heads):
                if w.layout == "BHND":
                    k[b, h, pos[b, h], :] *= mult
                else:
                    k[b, pos[b, h], h, :] *= mult
    if w.dtype == "bf16":
        qb, kb, vb = f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v)
        q, k, v = bf16_bits_to_f32(qb), bf16_bits_to_f32(kb), bf16_bits_to_f32(vb)
        return Inputs(w, q, k, v, qb, kb, vb, pos)
    if w.dtype != "f32":
        raise ValueError(f"unknown dtype {w.dtype!r}")
    return Inputs(w, q, k, v, None, None, None, pos)


def make_grad(w: Workload, seed_base: int | None = None):
    """The upstream gradient dO (shape and layout of Q) for the backward pass:
    N(0, 1) draws from seed 1000*cid+4 (or seed_base+4), rounded to bf16 for
    bf16 workloads.  Returns (float32 values, bf16 bits or None)."""
    base = 1000 * w.cid if seed_base is None else seed_base
    g = _draw(base + 4, w.q_shape(), 1.0)
    if w.dtype == "bf16":
        gb = f32_to_bf16_bits(g)
        return bf16_bits_to_f32(gb), gb
    return g, None


@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    """Decode attention over a paged KV cache: Nq new tokens per sequence
    attend to the sequence's L_b cached keys (the tokens sit at positions
    L_b - Nq .. L_b - 1; causal: token t sees keys j <= L_b - Nq + t)."""
    cid: int
    name: str
    B: int
    H: int
    Hkv: int
    Nq: int                 # new tokens per sequence
    max_len: int            # longest sequence (keys)
    min_len: int            # shortest sequence
    d: int
    block_size: int         # tokens per KV cache block
    causal: bool = False

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def max_blocks(self) -> int:
        return (self.max_len + self.block_size - 1) // self.block_size

    def scaled(self, **changes) -> "DecodeWorkload":
        return dataclasses.replace(self, **changes)


DECODE_WORKLOADS = {
    # one new token per sequence for a batch of 32 LLaMA-like (32 x 128) heads
    # with 8 KV heads, 4K-8K tokens cached in blocks of 16 ([nanhubrain]
    # "GatherPAKVCache": paged cache, block tables, GQA head selection)
    "decode_paged_gqa": DecodeWorkload(7, "decode_paged_gqa", 32, 32, 8, 1, 8192, 4096, 128, 16),
}


@dataclasses.dataclass
class PagedInputs:
    w: DecodeWorkload
    q: np.ndarray            # [B, Nq, H, d] float32 values
    k_cache: np.ndarray      # [num_blocks, block_size, Hkv, d] float32 values
    v_cache: np.ndarray
    q_bits: np.ndarray       # bf16 bits of the same
    k_bits: np.ndarray
    v_bits: np.ndarray
    seq_lens: np.ndarray     # [B] int32
    block_tables: np.ndarray  # [B, max_blocks] int32 physical block ids (-1: unused)


def make_paged(w: DecodeWorkload, seed_base: int | None = None) -> PagedInputs:
    """Seeded paged-cache inputs: sequence lengths uniform in [min_len,
    max_len] (seed +5); every sequence's blocks are distinct physical blocks
    of one cache, in a seeded random order (seed +6), with one spare block at
    the end of the cache that no table references; Q, K cache, V cache
    N(0, 1) (seeds +0, +1, +2), rounded to bf16."""
    base = 1000 * w.cid if seed_base is None else seed_base
    g = np.random.Generator(np.random.PCG64(base + 5))
    lens = g.integers(w.min_len, w.max_len + 1, size=w.B).astype(np.int32)
    nblk = (lens + w.block_size - 1) // w.block_size
    total = int(nblk.sum()) + 1
    perm = np.random.Generator(np.random.PCG64(base + 6)).permutation(total - 1).astype(np.int32)
    tables = np.full((w.B, w.max_blocks), -1, dtype=np.int32)
    at = 0
    for b in range(w.B):
        tables[b, :nblk[b]] = perm[at:at + nblk[b]]
        at += nblk[b]
    q = _draw(base + 0, (w.B, w.Nq, w.H, w.d), 1.0)
    kc = _draw(base + 1, (total, w.block_size, w.Hkv, w.d), 1.0)
    vc = _draw(base + 2, (total, w.block_size, w.Hkv, w.d), 1.0)
    qb, kb, vb = f32_to_bf16_bits(q), f32_to_bf16_bits(kc), f32_to_bf16_bits(vc)
    return PagedInputs(w, bf16_bits_to_f32(qb), bf16_bits_to_f32(kb), bf16_bits_to_f32(vb), qb, kb, vb,
                       lens, tables)


def sample_rows(w: Workload, n: int, seed: int = 7, peaked: np.ndarray | None = None) -> np.ndarray:
    """A sorted, de-duplicated sample of query rows for row-sampled checks:
    the first 16 and last 16 rows, up to 16 rows right after peaked keys of
    head (0, 0) when there are any, and seeded-uniform rows for the rest."""
    rows = set(range(min(16, w.Nq)))
    rows.update(range(max(0, w.Nq - 16), w.Nq))
    if peaked is not None:
        for p in peaked[0, 0][:16]:
            if p + 1 < w.Nq:
                rows.add(int(p) + 1)
    g = np.random.Generator(np.random.PCG64(seed))
    need = max(0, n - len(rows))
    if need:
        rows.update(int(x) for x in g.choice(w.Nq, size=min(need, w.Nq), replace=False))
    return np.array(sorted(rows), dtype=np.int32)


def tile_rows(w: Workload, per_tile: int, tile: int = 256, seed: int = 17,
              peaked: np.ndarray | None = None, n_edge: int = 16) -> np.ndarray:
    """A row table int32 [B*H, R] for row-sampled checks at full size, with
    rows of its own for every head (b, h) (table row b*H + h): the first and
    last ``n_edge`` rows, ``per_tile`` seeded-uniform rows inside every
    ``tile``-row block of queries (so every query tile of a launch is hit, at
    an offset that differs from head to head), and, when ``peaked`` key
    positions are given, the ``n_edge`` rows right after the first peaked
    keys of that head (K/V head h // (H / Hkv)), spread over its sorted list
    of peaked keys.  Entries may repeat."""
    g = np.random.Generator(np.random.PCG64(seed))
    n_tiles = (w.Nq + tile - 1) // tile
    starts = np.arange(n_tiles) * tile
    sizes = np.minimum(tile, w.Nq - starts)
    e = min(n_edge, w.Nq)
    table = []
    for bh in range(w.B * w.H):
        b, h = divmod(bh, w.H)
        rows = [np.arange(e), np.arange(w.Nq - e, w.Nq)]
        if peaked is not None:
            pk = peaked[b, h // (w.H // w.kv_heads)]
            pick = pk[np.linspace(0, pk.size - 1, n_edge).astype(np.int64)]
            rows.append(np.minimum(pick + 1, w.Nq - 1))
        offs = (g.random((per_tile, n_tiles)) * sizes).astype(np.int64)
        rows.append((starts + offs).reshape(-1))
        table.append(np.concatenate(rows))
    return np.stack(table).astype(np.int32)

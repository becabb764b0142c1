"""GPU parity of the block-sparse backward pass (fa_bwd_sparse through the C
ABI binding) against the numpy fp64 oracle (oracle.sparse.
attn_bwd_block_sparse) on seeded inputs, at the elementwise bound of
tests/test_gpu_bwd.py taken over each row's visible keys (gpu_common.
bwd_bounds).  Rows that see no key must give dQ = 0 exactly.

Cases: random masks of several densities (256-query x 64-key blocks) in
both layouts, causal or not, d = 64 and 128, ragged last blocks; masks with
an empty query block and a key block no query sees; the all-ones mask
(equal to the dense backward); the pipeline through the GPU block-sparse
forward; and the full-size BigBird workload on sampled rows of one head."""
import numpy as np
import pytest

from oracle import sparse
from exact_attention_112_amd import inputs as I
from gpu_common import bwd_bounds, check_bound, log, require_gpu

pytestmark = pytest.mark.gpu

BQ, BK = I.SPARSE_BQ, I.SPARSE_BK
W = I.WORKLOADS
BASE = W["selfattn_b4h32n8k"]
PRE = W["llama_prefill_causal"]


def _t(bits):
    import torch
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to("cuda")


def _bhnd(x, layout):
    return x if layout == "BHND" else x.transpose(0, 2, 1, 3)


def _random_mask(w, density, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    shape = (w.B, w.H, (w.Nq + BQ - 1) // BQ, (w.Nk + BK - 1) // BK)
    return (g.random(shape) < density).astype(np.uint8)


def _run(w, mask, *, use_gpu_forward=False, qrows=None, krows=None, heads=None):
    import torch
    import exact_attention_112_amd as fa

    require_gpu()
    log(f"case bwd_sparse {w.name} B{w.B} H{w.H} Nq{w.Nq} Nk{w.Nk} d{w.d} {w.layout} causal={w.causal} "
        f"density={mask.mean():.3f} gpu_fwd={use_gpu_forward}")
    inp = I.make_inputs(w)
    do_vals, do_bits = I.make_grad(w)
    tq, tk, tv, tdo = (_t(x) for x in (inp.q_bits, inp.k_bits, inp.v_bits, do_bits))
    tmask = torch.from_numpy(mask).to("cuda")
    Q, K, V, G = (_bhnd(x, w.layout) for x in (inp.q, inp.k, inp.v, do_vals))
    heads = heads or [(b, h) for b in range(w.B) for h in range(w.H)]
    if use_gpu_forward:
        o_t, lse_t = fa.fwd(tq, tk, tv, causal=w.causal, scale=w.scale, layout=w.layout, block_mask=tmask)
    else:
        o_ref = np.zeros((w.B, w.H, w.Nq, w.d))
        lse_ref = np.full((w.B, w.H, w.Nq), -np.inf)
        for b in range(w.B):
            for h in range(w.H):
                o_ref[b, h], lse_ref[b, h] = sparse.attn_fwd_block_sparse(
                    Q[b, h], K[b, h], V[b, h], mask[b, h], bq=BQ, bk=BK, scale=w.scale, causal=w.causal)
        o_st = o_ref if w.layout == "BHND" else o_ref.transpose(0, 2, 1, 3)
        o_t = torch.from_numpy(np.ascontiguousarray(o_st, dtype=np.float32)).to("cuda")
        lse_t = torch.from_numpy(lse_ref.astype(np.float32)).to("cuda")
    dq, dk, dv = fa.bwd(tq, tk, tv, o_t, tdo, lse_t, causal=w.causal, scale=w.scale, layout=w.layout,
                        block_mask=tmask)
    torch.cuda.synchronize()
    dq, dk, dv = (_bhnd(x.cpu().numpy().astype(np.float64), w.layout) for x in (dq, dk, dv))
    O = _bhnd(o_t.float().cpu().numpy().astype(np.float64), w.layout)
    L = lse_t.cpu().numpy().astype(np.float64)
    qr = np.arange(w.Nq) if qrows is None else np.asarray(qrows)
    kr = np.arange(w.Nk) if krows is None else np.asarray(krows)
    for b, h in heads:
        mk = mask[b, h]
        f64 = lambda x: x[b, h].astype(np.float64)
        rq, rk, rv = sparse.attn_bwd_block_sparse(Q[b, h], K[b, h], V[b, h], G[b, h], mk, bq=BQ, bk=BK,
                                                  scale=w.scale, causal=w.causal, qrows=qr, krows=kr)
        o_h, lse_h = sparse.attn_fwd_block_sparse(Q[b, h], K[b, h], V[b, h], mk, bq=BQ, bk=BK, scale=w.scale,
                                                  causal=w.causal)

        def visible(rows, cols):
            m = mk[rows[:, None] // BQ, cols[None, :] // BK] != 0
            if w.causal:
                m &= cols[None, :] <= rows[:, None]
            return m

        bq, bk, bv = bwd_bounds(f64(Q), f64(K), f64(V), f64(G), o_h, lse_h, O[b, h], L[b, h], w.scale,
                                visible, qr, kr)
        log(f"  head ({b},{h})")
        check_bound("dQ", dq[b, h, qr], rq, bq)
        check_bound("dK", dk[b, h, kr], rk, bk)
        check_bound("dV", dv[b, h, kr], rv, bv)
        empty = ~np.isfinite(lse_h[qr])
        assert np.all(dq[b, h, qr][empty] == 0.0), "rows without keys must give dQ = 0"


CASES = {
    "bhnd_d128": (BASE.scaled(B=1, H=2, Nq=600, Nk=700), 0.4),
    "bsnd_causal_d128": (PRE.scaled(H=2, Nq=777, Nk=777), 0.5),
    "bhnd_d64_dense_half": (BASE.scaled(B=2, H=1, Nq=520, Nk=300, d=64), 0.6),
    "bhnd_causal_d64_sparse": (BASE.scaled(B=1, H=2, Nq=1030, Nk=1030, d=64, causal=True), 0.25),
}


@pytest.mark.parametrize("name", list(CASES))
def test_bwd_sparse_every_element(name):
    w, dens = CASES[name]
    _run(w, _random_mask(w, dens, seed=len(name) * 101))


def test_bwd_sparse_empty_blocks():
    w = BASE.scaled(B=1, H=2, Nq=700, Nk=500)
    mask = _random_mask(w, 0.7, seed=5)
    mask[:, :, 1, :] = 0          # query block 1 sees no key
    mask[:, :, :, 3] = 0          # key block 3 is seen by no query
    _run(w, mask)


def test_bwd_sparse_all_ones_equals_dense():
    import torch
    import exact_attention_112_amd as fa

    require_gpu()
    w = PRE.scaled(H=2, Nq=333, Nk=333)
    inp = I.make_inputs(w)
    _, do_bits = I.make_grad(w)
    tq, tk, tv, tdo = (_t(x) for x in (inp.q_bits, inp.k_bits, inp.v_bits, do_bits))
    o, lse = fa.fwd(tq, tk, tv, causal=True, scale=w.scale, layout=w.layout)
    ones = torch.ones((w.B, w.H, (w.Nq + BQ - 1) // BQ, (w.Nk + BK - 1) // BK), dtype=torch.uint8, device="cuda")
    a = fa.bwd(tq, tk, tv, o, tdo, lse, causal=True, scale=w.scale, layout=w.layout)
    b = fa.bwd(tq, tk, tv, o, tdo, lse, causal=True, scale=w.scale, layout=w.layout, block_mask=ones)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y), "an all-ones mask must give the dense backward bit for bit"


def test_bwd_sparse_through_gpu_forward():
    w = BASE.scaled(B=1, H=2, Nq=900, Nk=1100)
    _run(w, _random_mask(w, 0.35, seed=9), use_gpu_forward=True)


def test_bwd_sparse_full_size_sampled():
    w = W["sparse_bigbird"]
    mask = I.make_block_mask(w)
    kr = np.array([0, 63, 64, 5000, 12345, 16383])
    qr = np.array([0, 255, 256, 7000, 16383, 9999])
    _run(w, mask, use_gpu_forward=True, qrows=qr, krows=kr, heads=[(1, 7)])

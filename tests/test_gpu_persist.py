"""GPU parity of the persistent forward kernel (plain non-causal attention
over whole key tiles, at least two query tiles per CU), element by element
against the fp64 oracle: the shapes below make fa_fwd take that kernel
(Nk a multiple of 128 and more than 128; at least 512 query tiles of 256
rows), with query tiles of several heads per workgroup, a ragged last query
tile, a head count that is not a multiple of 8, both layouts, d = 64 and
bf16 output.
"""
import numpy as np
import pytest

import oracle
from exact_attention_112_amd import inputs as I
from gpu_common import check, errors, log, require_gpu, run_gpu, to_bhnd, tol_for, upload

pytestmark = pytest.mark.gpu

BASE = I.WORKLOADS["selfattn_b4h32n8k"]

CASES = {
    # 32 query tiles x 16 heads = 512 (two per CU), 16 key tiles
    "b1h16_n8192_k1024": BASE.scaled(B=1, H=16, Nq=8192, Nk=1024),
    # 32 x 19 = 608 query tiles (two or three per workgroup), the last query
    # tile ragged (8000 rows), BSND, a head count that is not a multiple of 8
    "b1h19_n8000_k640_bsnd": BASE.scaled(B=1, H=19, Nq=8000, Nk=640, layout="BSND"),
    # d = 64, four key tiles
    "b2h8_n8192_k256_d64": BASE.scaled(B=2, H=8, Nq=8192, Nk=256, d=64),
}


@pytest.mark.parametrize("name", list(CASES))
def test_persistent_kernel_full_compare(name):
    _compare(CASES[name])


def test_persistent_kernel_bf16_output():
    import torch
    _compare(CASES["b1h16_n8192_k1024"], out_dtype=torch.bfloat16)


def _compare(w, out_dtype=None):
    import torch
    require_gpu()
    log(f"case {w.name} B{w.B} H{w.H} Nq{w.Nq} Nk{w.Nk} d{w.d} {w.layout} out={out_dtype}")
    inp = I.make_inputs(w)
    tq, tk, tv = upload(inp)
    o, lse = run_gpu(w, tq, tk, tv, out_dtype=out_dtype)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attn_fwd(inp.q, inp.k, inp.v, scale=w.scale, causal=w.causal, layout=w.layout)
    err = errors(to_bhnd(o, w.layout), lse.cpu().numpy().astype(np.float64), o_ref, lse_ref)
    check(err, tol_for(w, out_dtype), w.name)

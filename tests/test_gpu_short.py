"""GPU parity of the short-key forward kernel (bf16, at most 128 keys, no
band or block mask: every such call of fa_fwd / fa_fwd_ex runs it) against
the fp64 oracle, element by element, at the forward tolerances (O max-abs
1e-2, mean-abs 1e-3, LSE max-abs 1e-3; bf16 O at the bf16-output bound).

Cases: key counts at and around the kernel's 32-key blocks (1, 31, 32, 33,
96, 97, 128); d = 64 and 128; causal or not; both layouts; grouped KV heads
(GQA, MQA); bf16 output; query counts that leave a ragged last tile and a
partly filled last workgroup, with several query tiles per wave (the one-
tile-ahead Q loads alternate their two LDS stages); and the
Stable-Diffusion cross-attention workload at full size (Nk = 77) in the
bench's launch configuration."""
import numpy as np
import pytest

import oracle
from exact_attention_112_amd import inputs as I
from gpu_common import BF16_OUT_TOL, BF16_TOL, check, errors, log, require_gpu, to_bhnd, upload

pytestmark = pytest.mark.gpu

W = I.WORKLOADS
X = W["sd_crossattn"]


def _run(w, out_bf16=False):
    import torch
    import exact_attention_112_amd as fa

    require_gpu()
    log(f"case short {w.name} B{w.B} H{w.H} Hkv{w.kv_heads} Nq{w.Nq} Nk{w.Nk} d{w.d} {w.layout} "
        f"causal={w.causal} out_bf16={out_bf16}")
    inp = I.make_inputs(w)
    tq, tk, tv = upload(inp)
    o, lse = fa.fwd(tq, tk, tv, causal=w.causal, scale=w.scale, layout=w.layout,
                    out_dtype=torch.bfloat16 if out_bf16 else torch.float32)
    torch.cuda.synchronize()
    if w.kv_heads == w.H:
        o_ref, lse_ref = oracle.attn_fwd(inp.q, inp.k, inp.v, scale=w.scale, causal=w.causal, layout=w.layout)
    else:
        o_ref, lse_ref = oracle.attn_fwd_ex(inp.q, inp.k, inp.v, scale=w.scale, causal=w.causal, layout=w.layout)
    err = errors(to_bhnd(o, w.layout), lse.cpu().numpy().astype(np.float64), o_ref, lse_ref)
    check(err, BF16_OUT_TOL if out_bf16 else BF16_TOL, w.name)


@pytest.mark.parametrize("nk", [1, 31, 32, 33, 96, 97, 128])
@pytest.mark.parametrize("d", [64, 128])
def test_short_key_counts(nk, d):
    _run(X.scaled(B=1, H=3, Nq=333, Nk=nk, d=d))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("layout", ["BHND", "BSND"])
def test_short_causal_layouts(causal, layout):
    _run(I.Workload(93, "short", 2, 3, 300, 100, 128, "bf16", layout, causal))
    _run(I.Workload(94, "short64", 1, 2, 250, 70, 64, "bf16", layout, causal))


def test_short_grouped_heads():
    _run(X.scaled(B=1, H=8, Hkv=2, Nq=700, Nk=77))
    _run(I.Workload(95, "short_mqa", 1, 4, 400, 120, 128, "bf16", "BSND", True, Hkv=1))


def test_short_bf16_output():
    _run(X.scaled(B=1, H=2, Nq=515, Nk=77), out_bf16=True)


def test_short_several_tiles_per_wave():
    # 8 heads x 129 row blocks of 128 > 1024: two tiles per wave and a last
    # workgroup with only 37 rows
    _run(X.scaled(B=1, H=8, Nq=16384 + 37, Nk=128, d=128))


def test_short_full_size_crossattn():
    _run(X)

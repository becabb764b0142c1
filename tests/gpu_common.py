"""Helpers shared by the GPU tests: upload seeded inputs, run the HIP path
through the C ABI binding, compare with the oracle at the stated tolerances."""
from __future__ import annotations

import sys

import numpy as np
import pytest

from exact_attention_112_amd import inputs as I

# Tolerances: O max-abs 1e-2 and mean-abs 1e-3, LSE max-abs 1e-3 for bf16
# inputs (O compared in fp32 against the fp64 oracle); 1e-5 for fp32 inputs.
BF16_TOL = dict(o_max=1e-2, o_mean=1e-3, lse_max=1e-3)
F32_TOL = dict(o_max=1e-5, o_mean=1e-5, lse_max=1e-5)
# bf16 *output* adds up to half a bf16 ulp of |O| (2^-9 relative): not part of
# the parity bar, checked with this wider bound.
BF16_OUT_TOL = dict(o_max=2.5e-2, o_mean=3e-3, lse_max=1e-3)


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def require_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a GPU")


def upload(inp: I.Inputs):
    import torch
    if inp.w.dtype == "bf16":
        f = lambda bits: torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to("cuda")
        return f(inp.q_bits), f(inp.k_bits), f(inp.v_bits)
    f = lambda x: torch.from_numpy(x).to("cuda")
    return f(inp.q), f(inp.k), f(inp.v)


def run_gpu(w: I.Workload, tq, tk, tv, *, out_dtype=None, scale=None):
    import exact_attention_112_amd as fa
    return fa.fwd(tq, tk, tv, causal=w.causal, scale=w.scale if scale is None else scale,
                  layout=w.layout, out_dtype=out_dtype)


def to_bhnd(o, layout):
    """GPU O in the workload layout -> float64 numpy [B,H,N,d]."""
    a = o.float().cpu().numpy().astype(np.float64)
    return a if layout == "BHND" else a.transpose(0, 2, 1, 3)


def errors(o_gpu, lse_gpu, o_ref, lse_ref):
    do = np.abs(o_gpu - o_ref)
    dl = np.abs(lse_gpu - lse_ref)
    return dict(o_max=float(do.max()), o_mean=float(do.mean()), lse_max=float(dl.max()),
                finite=bool(np.isfinite(o_gpu).all() and np.isfinite(lse_gpu).all()))


def check(err, tol, what=""):
    log(f"  {what}: O max {err['o_max']:.3e} mean {err['o_mean']:.3e}  LSE max {err['lse_max']:.3e}")
    assert err["finite"], f"{what}: non-finite output"
    assert err["o_max"] <= tol["o_max"], f"{what}: O max-abs {err['o_max']} > {tol['o_max']}"
    assert err["o_mean"] <= tol["o_mean"], f"{what}: O mean-abs {err['o_mean']} > {tol['o_mean']}"
    assert err["lse_max"] <= tol["lse_max"], f"{what}: LSE max-abs {err['lse_max']} > {tol['lse_max']}"


def tol_for(w: I.Workload, out_dtype=None):
    import torch
    if w.dtype == "f32":
        return F32_TOL
    return BF16_OUT_TOL if out_dtype == torch.bfloat16 else BF16_TOL


def bwd_bounds(q, k, v, do, o_ref, lse_ref, o_given, lse_given, scale, visible, qrows, krows):
    """Elementwise error bounds of the backward pass for one head (the bound
    tests/test_gpu_bwd.py derives: P and dS rounded to bf16, u = 2^-8, fp32
    sums eps = 1e-5, and the exact effect of the O and LSE the backward is
    given), over the pairs visible(rows, cols) marks.  q, do, o_* [Nq, d];
    k, v [Nk, d]; lse_* [Nq] (float64).  Returns (bq [RQ,d], bk [RK,d],
    bv [RK,d])."""
    u, eps = 2.0 ** -8, 1e-5
    Nq, Nk = q.shape[0], k.shape[0]
    live = np.isfinite(lse_ref)
    lse = np.where(live, lse_ref, 0.0)
    D = np.sum(do * o_ref, axis=1)
    Dabs = np.sum(np.abs(do * o_ref), axis=1)
    dD = np.abs(np.sum(do * (o_given - o_ref), axis=1))
    dL = np.where(live, np.expm1(np.abs(np.where(live, lse_given, 0.0) - lse) + 1e-7 * np.abs(lse)), 0.0)

    def ds_err(rows_q, cols_k):
        s = scale * (q[rows_q] @ k[cols_k].T)
        p = np.where(visible(rows_q, cols_k), np.exp(np.minimum(s - lse[rows_q, None], 80.0)), 0.0)
        dp = do[rows_q] @ v[cols_k].T
        dp_abs = np.abs(do[rows_q]) @ np.abs(v[cols_k]).T
        ds = p * (dp - D[rows_q, None])
        e = (u + dL[rows_q, None]) * np.abs(ds) + p * (eps * (dp_abs + Dabs[rows_q, None]) + dD[rows_q, None])
        return e, p

    allq, allk = np.arange(Nq), np.arange(Nk)
    eq, _ = ds_err(np.asarray(qrows), allk)
    bq = scale * (eq @ np.abs(k))
    ek, pk = ds_err(allq, np.asarray(krows))
    bk = scale * (ek.T @ np.abs(q))
    bv = (pk * (u + eps + dL[:, None])).T @ np.abs(do)
    return bq, bk, bv


def check_bound(name, got, ref, bound):
    """|got - ref| <= 1.1 x bound + 1e-5 x max|ref| elementwise, and finite."""
    err = np.abs(got - ref)
    slack = 1e-5 * max(1e-30, float(np.max(np.abs(ref))))
    ratio = float(np.max(err / (1.1 * bound + slack)))
    rel = float(np.max(err) / max(1e-30, np.max(np.abs(ref))))
    log(f"    {name}: max|err| {np.max(err):.3e} (rel {rel:.2e})  max err/bound {ratio:.3f}")
    assert np.isfinite(got).all(), f"{name}: non-finite"
    assert ratio <= 1.0, f"{name}: error exceeds its bound (ratio {ratio:.3f})"

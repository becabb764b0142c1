"""Host emulation of the forward kernel's rounding of P (no GPU): the scores of
each 64-key tile in fp32, P = exp2(s*scale*log2e - m) in fp32, P rounded to bf16
(round to nearest even) for the P V product, fp32 row sums, and the lane halves
of a tile (keys whose offset in their group of 8 is below 4, and the rest).

Three ways to keep the running max m are compared against the exact softmax
attention (fp64) on rows with peaked keys (1 % of the keys scaled by 8, the
long-context workload's recipe):
  * eager: m follows every increase, so the row's largest key has p = 1;
  * lazy: m moves only when a tile max exceeds it by more than tau (log2 units);
  * lazy + rounding term: as lazy, and the normaliser of O adds bf16(p) - p of
    each lane half's largest p per tile (what the kernel does, tau = 4).
The LSE always comes from the unrounded sum.  The online-softmax merge these
schemes run is the one of [nanhubrain] "online softmax mathematics"; the
pages do not fix the rounding of P, so this pins the reading the kernel takes.
"""
import numpy as np
import pytest

N, D, T = 8192, 128, 64


def _bf16(x):
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


def _inputs(seed=7, rows=1024):
    rng = np.random.default_rng(seed)
    q = _bf16(rng.standard_normal((rows, D)))
    k = rng.standard_normal((N, D))
    k[rng.choice(N, N // 100, replace=False)] *= 8
    k = _bf16(k)
    v = _bf16(rng.standard_normal((N, D)))
    return q, k, v


def _emulate(q, k, v, scheme, tau):
    scale = 1.0 / np.sqrt(D)
    sl2 = np.float32(scale * np.log2(np.e))
    S = (q.astype(np.float64) @ k.T.astype(np.float64)).astype(np.float32)
    x64 = S.astype(np.float64) * scale
    mx = x64.max(1, keepdims=True)
    P = np.exp(x64 - mx)
    o_ex = (P @ v.astype(np.float64)) / P.sum(1)[:, None]
    lse_ex = mx[:, 0] + np.log(P.sum(1))
    R = q.shape[0]
    m = np.full(R, -np.inf, np.float32)
    l = np.zeros(R, np.float32)
    dl = np.zeros(R, np.float32)
    o = np.zeros((R, D), np.float32)
    half = (np.arange(T) % 8) >= 4
    for t in range(N // T):
        s = S[:, t * T:(t + 1) * T]
        mt = (s.max(1).astype(np.float64) * float(sl2)).astype(np.float32)
        if scheme == "eager":
            moved = mt > m
            if moved.any():
                m_new = np.where(moved, mt, m)
                alpha = np.where(np.isfinite(m), np.exp2(m - m_new), 0).astype(np.float32)
                l, dl, o, m = l * alpha, dl * alpha, o * alpha[:, None], m_new
        elif (mt > m + tau).any():
            m_new = np.maximum(mt, m)
            alpha = np.where(np.isfinite(m), np.exp2(m - m_new), 0).astype(np.float32)
            l, dl, o, m = l * alpha, dl * alpha, o * alpha[:, None], m_new
        e = np.exp2((s.astype(np.float64) * float(sl2) - m[:, None]).astype(np.float32))
        l = l + e.sum(1, dtype=np.float32)
        if scheme == "lazy_fix":
            for sel in (half, ~half):
                em = np.exp2((s[:, sel].max(1).astype(np.float64) * float(sl2) - m).astype(np.float32))
                dl = dl + (_bf16(em) - em)
        o = o + (_bf16(e).astype(np.float64) @ v[t * T:(t + 1) * T].astype(np.float64)).astype(np.float32)
    o_k = o / (l + dl)[:, None]
    lse_k = (m.astype(np.float64) + np.log2(l.astype(np.float64))) * np.log(2.0)
    return np.abs(o_k - o_ex).max(), np.abs(lse_k - lse_ex).max()


@pytest.fixture(scope="module")
def errs():
    q, k, v = _inputs()
    return {name: _emulate(q, k, v, name, tau) for name, tau in
            (("eager", 0.0), ("lazy", 8.0), ("lazy_fix", 4.0))}


def test_kernel_scheme_within_the_bar_with_margin(errs):
    o_err, lse_err = errs["lazy_fix"]
    assert o_err < 5e-3, o_err          # the bar is 1e-2
    assert lse_err < 1e-4, lse_err      # the bar is 1e-3


def test_rounding_term_matters(errs):
    # without the rounding term the stale max costs accuracy on peaked rows;
    # with it the error is back at the eager max's level
    assert errs["lazy"][0] > 1.3 * errs["lazy_fix"][0], errs
    assert errs["lazy_fix"][0] < 1.3 * errs["eager"][0], errs

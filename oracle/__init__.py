"""CPU oracle for the attention forward and backward passes -- TEST
INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never calls it, and
it shares no code with the GPU path (the only common module is the seeded
input generator, which holds none of the method's arithmetic).

Five implementations live here (plus the paged-cache and block-sparse
references in paged.py and sparse.py):

* ``attn_fwd`` -- the plain definition, a two-pass fp64 softmax attention in C
  (``oracle.c``): scores, row max, exp-sum, weighted sum of values, one row at
  a time.  It follows [nanhubrain] "exact source of the quadratic memory"
  (S = QK^T/sqrt(d), P = softmax(S), O = PV), [nanhubrain] "online softmax
  mathematics" (max-subtracted softmax) and [ascendai] section 6.1 (causal:
  strict upper triangle masked, key j visible to query i iff j <= i).
* ``attn_bwd`` -- the gradients dQ, dK, dV of the same attention for an
  upstream gradient dO, by their plain definition in fp64 C (``oracle.c``):
  P, dP = dO V^T, D_i = rowsum(P * dP) over the whole row, dS = P * (dP - D),
  dQ = scale dS K, dK = scale dS^T Q, dV = P^T dO ([nanhubrain] "backward
  recomputation", with the row term taken over the whole row).
* ``attn_fwd_ex`` -- the forward with grouped key/value heads (GQA/MQA:
  query head h reads KV head h // (H // Hkv), [nanhubrain] "GatherPAKVCache")
  and a band of visible keys i-left <= j <= i+right ([pwwt] "standard vs
  IO-aware": pre_tokens / next_tokens), plain fp64 C; a row with no visible
  key gives O = 0, LSE = -inf.
* ``attn_bwd_ex`` -- the gradients of ``attn_fwd_ex``: those of ``attn_bwd``
  over each row's visible keys, with dK and dV of a KV head summed over the
  query heads that read it; plain fp64 C.
* ``online.attn_fwd_online`` -- the pages' own algorithm, the tiled forward
  with the online-softmax recurrence ([nanhubrain] "tiling skeleton",
  [ascendai] section 2.2), in numpy fp64, over caller-chosen block splits.

``paged.gather_paged_kv`` / ``paged.decode_reference`` (numpy) gather a
paged KV cache the way [nanhubrain] "GatherPAKVCache" describes (logical block
-> physical block through the block table, optional KV head selection) and
run ``attn_fwd_ex`` on the gathered sequence for decode attention.

Page key: [nanhubrain] = nanhubrain.csdn.net (FlashAttention in CANN
ops-transformer), [pwwt] = www.pwwt.cn/news/2518640, [ascendai] =
ascendai.csdn.net (efficient attention in CANN ops-nn).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "oracle.c")
LIBRARY = os.path.join(_HERE, "liboracle.so")

_c_i64 = ctypes.c_int64
_c_int = ctypes.c_int
_c_dbl = ctypes.c_double
_c_ptr = ctypes.c_void_p


def build(source: str = SOURCE, output: str = LIBRARY) -> str:
    """Compile ``oracle.c`` with gcc (plain -O2, no fast-math) into a shared library."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-Wall", "-Wextra", "-o", output, source, "-lm"]
    subprocess.run(cmd, check=True)
    return output


class OracleLib:
    """ctypes view of one compiled oracle library (the default, or a test variant)."""

    def __init__(self, path: str = LIBRARY):
        if not os.path.exists(path):
            raise FileNotFoundError(
                f"oracle library {path} is not built; run oracle.build() first")
        self.path = path
        self._lib = ctypes.CDLL(path)
        f = self._lib.oracle_attn_fwd
        f.restype = _c_int
        f.argtypes = ([_c_ptr] * 3 + [_c_i64] * 9 + [_c_int] * 5 + [_c_dbl, _c_int]
                      + [_c_ptr, _c_int, _c_ptr, _c_ptr, _c_int])
        f2 = self._lib.oracle_attn_fwd_rowtab
        f2.restype = _c_int
        f2.argtypes = f.argtypes
        g = self._lib.oracle_attn_probs
        g.restype = _c_int
        g.argtypes = [_c_ptr, _c_ptr, _c_i64, _c_i64, _c_int, _c_int, _c_int,
                      _c_dbl, _c_int, _c_ptr]
        h = self._lib.oracle_attn_bwd
        h.restype = _c_int
        h.argtypes = ([_c_ptr] * 4 + [_c_i64] * 6 + [_c_int] * 5 + [_c_dbl, _c_int]
                      + [_c_ptr, _c_int, _c_ptr, _c_int, _c_ptr, _c_ptr, _c_ptr, _c_int])
        x = self._lib.oracle_attn_fwd_ex
        x.restype = _c_int
        x.argtypes = ([_c_ptr] * 3 + [_c_i64] * 6 + [_c_int] * 6 + [_c_dbl] + [_c_int] * 3
                      + [_c_ptr, _c_int, _c_ptr, _c_ptr, _c_int])
        y = self._lib.oracle_attn_bwd_ex
        y.restype = _c_int
        y.argtypes = ([_c_ptr] * 4 + [_c_i64] * 6 + [_c_int] * 6 + [_c_dbl] + [_c_int] * 3
                      + [_c_ptr, _c_int, _c_ptr, _c_int, _c_ptr, _c_ptr, _c_ptr, _c_int])
        self._lib.oracle_max_threads.restype = _c_int

    def max_threads(self) -> int:
        return int(self._lib.oracle_max_threads())

    def attn_fwd(self, q, k, v, *, scale: float, causal: bool = False,
                 layout: str = "BHND", rows=None, n_threads: int = 0):
        """O [B,H,R,d] and LSE [B,H,R] in float64.

        q, k, v: float32 arrays in the layout's storage shape -- ``BHND`` is
        [B,H,N,d], ``BSND`` is [B,N,H,d].  ``rows``: optional query indices
        (the same for every (b,h)), or a 2-D table [B*H, R] that gives each
        head (b, h) its own R rows (row b*H + h); default all rows.  ``scale``
        is used as given (no default resolution here).
        """
        q = np.ascontiguousarray(q, dtype=np.float32)
        k = np.ascontiguousarray(k, dtype=np.float32)
        v = np.ascontiguousarray(v, dtype=np.float32)
        if layout == "BHND":
            B, H, Nq, d = q.shape
            Nk = k.shape[2]
            qs = (H * Nq * d, Nq * d, d)
            ks = (H * Nk * d, Nk * d, d)
        elif layout == "BSND":
            B, Nq, H, d = q.shape
            Nk = k.shape[1]
            qs = (Nq * H * d, d, H * d)
            ks = (Nk * H * d, d, H * d)
        else:
            raise ValueError(f"unknown layout {layout!r}")
        if k.shape != v.shape:
            raise ValueError("k and v must have the same shape")
        if rows is None:
            R = Nq
            rows_arr = None
            rows_ptr = None
        else:
            rows_arr = np.ascontiguousarray(rows, dtype=np.int32)
            if rows_arr.ndim == 2 and rows_arr.shape[0] != B * H:
                raise ValueError("a row table needs one row of indices per (b, h)")
            R = int(rows_arr.shape[-1])
            rows_ptr = rows_arr.ctypes.data
        o = np.empty((B, H, R, d), dtype=np.float64)
        lse = np.empty((B, H, R), dtype=np.float64)
        fn = self._lib.oracle_attn_fwd_rowtab if rows is not None and rows_arr.ndim == 2 else self._lib.oracle_attn_fwd
        rc = fn(
            q.ctypes.data, k.ctypes.data, v.ctypes.data,
            *qs, *ks, *ks, B, H, Nq, Nk, d, float(scale), int(bool(causal)),
            rows_ptr, R, o.ctypes.data, lse.ctypes.data, int(n_threads))
        if rc != 0:
            raise RuntimeError(f"oracle_attn_fwd failed with code {rc}")
        return o, lse

    def attn_bwd(self, q, k, v, do, *, scale: float, causal: bool = False,
                 layout: str = "BHND", qrows=None, krows=None, want_dq: bool = True,
                 want_dkv: bool = True, n_threads: int = 0):
        """(dQ [B,H,RQ,d], dK [B,H,RK,d], dV [B,H,RK,d]) in float64 (None for
        the parts not asked for).

        q, k, v, do: float32 arrays in the layout's storage shape (do has q's
        shape).  ``qrows`` / ``krows``: optional query / key indices (the same
        for every (b, h)); default all rows.
        """
        q = np.ascontiguousarray(q, dtype=np.float32)
        k = np.ascontiguousarray(k, dtype=np.float32)
        v = np.ascontiguousarray(v, dtype=np.float32)
        do = np.ascontiguousarray(do, dtype=np.float32)
        if q.shape != do.shape or k.shape != v.shape:
            raise ValueError("do must have q's shape and v k's shape")
        if layout == "BHND":
            B, H, Nq, d = q.shape
            Nk = k.shape[2]
            qs = (H * Nq * d, Nq * d, d)
            ks = (H * Nk * d, Nk * d, d)
        elif layout == "BSND":
            B, Nq, H, d = q.shape
            Nk = k.shape[1]
            qs = (Nq * H * d, d, H * d)
            ks = (Nk * H * d, d, H * d)
        else:
            raise ValueError(f"unknown layout {layout!r}")

        def idx(rows, n):
            if rows is None:
                return None, None, n
            a = np.ascontiguousarray(rows, dtype=np.int32)
            return a, a.ctypes.data, int(a.size)

        qa, qp, RQ = idx(qrows, Nq)
        ka, kp, RK = idx(krows, Nk)
        dq = np.empty((B, H, RQ, d), dtype=np.float64) if want_dq else None
        dk = np.empty((B, H, RK, d), dtype=np.float64) if want_dkv else None
        dv = np.empty((B, H, RK, d), dtype=np.float64) if want_dkv else None
        ptr = lambda a: None if a is None else a.ctypes.data
        rc = self._lib.oracle_attn_bwd(
            q.ctypes.data, k.ctypes.data, v.ctypes.data, do.ctypes.data,
            *qs, *ks, B, H, Nq, Nk, d, float(scale), int(bool(causal)),
            qp, RQ, kp, RK, ptr(dq), ptr(dk), ptr(dv), int(n_threads))
        if rc != 0:
            raise RuntimeError(f"oracle_attn_bwd failed with code {rc}")
        return dq, dk, dv

    def attn_fwd_ex(self, q, k, v, *, scale: float, causal: bool = False, window=(-1, -1),
                    layout: str = "BHND", rows=None, n_threads: int = 0):
        """O [B,H,R,d] and LSE [B,H,R] (float64) with grouped KV heads and a band.

        q: [B,H,Nq,d] (BHND) or [B,Nq,H,d] (BSND); k, v: the same with Nk and
        Hkv heads (H % Hkv == 0; query head h reads KV head h // (H // Hkv)).
        window = (left, right): key j visible to query i iff i-left <= j <=
        i+right (a negative bound is unbounded), and j <= i if causal.  Rows
        with no visible key give O = 0 and LSE = -inf.
        """
        q = np.ascontiguousarray(q, dtype=np.float32)
        k = np.ascontiguousarray(k, dtype=np.float32)
        v = np.ascontiguousarray(v, dtype=np.float32)
        if k.shape != v.shape:
            raise ValueError("k and v must have the same shape")
        if layout == "BHND":
            B, H, Nq, d = q.shape
            Hkv, Nk = k.shape[1], k.shape[2]
            qs = (H * Nq * d, Nq * d, d)
            ks = (Hkv * Nk * d, Nk * d, d)
        elif layout == "BSND":
            B, Nq, H, d = q.shape
            Nk, Hkv = k.shape[1], k.shape[2]
            qs = (Nq * H * d, d, H * d)
            ks = (Nk * Hkv * d, d, Hkv * d)
        else:
            raise ValueError(f"unknown layout {layout!r}")
        if rows is None:
            R, rows_arr, rows_ptr = Nq, None, None
        else:
            rows_arr = np.ascontiguousarray(rows, dtype=np.int32)
            R, rows_ptr = int(rows_arr.size), rows_arr.ctypes.data
        o = np.empty((B, H, R, d), dtype=np.float64)
        lse = np.empty((B, H, R), dtype=np.float64)
        rc = self._lib.oracle_attn_fwd_ex(
            q.ctypes.data, k.ctypes.data, v.ctypes.data, *qs, *ks, B, H, Hkv, Nq, Nk, d,
            float(scale), int(bool(causal)), int(window[0]), int(window[1]),
            rows_ptr, R, o.ctypes.data, lse.ctypes.data, int(n_threads))
        if rc != 0:
            raise RuntimeError(f"oracle_attn_fwd_ex failed with code {rc}")
        return o, lse

    def attn_bwd_ex(self, q, k, v, do, *, scale: float, causal: bool = False, window=(-1, -1),
                    layout: str = "BHND", qrows=None, krows=None, want_dq: bool = True,
                    want_dkv: bool = True, n_threads: int = 0):
        """(dQ [B,H,RQ,d], dK [B,Hkv,RK,d], dV [B,Hkv,RK,d]) in float64 with
        grouped KV heads and a band (as ``attn_fwd_ex``); None for the parts
        not asked for.  q and do have H heads, k and v Hkv heads; ``qrows`` /
        ``krows`` as in ``attn_bwd``.
        """
        q = np.ascontiguousarray(q, dtype=np.float32)
        k = np.ascontiguousarray(k, dtype=np.float32)
        v = np.ascontiguousarray(v, dtype=np.float32)
        do = np.ascontiguousarray(do, dtype=np.float32)
        if q.shape != do.shape or k.shape != v.shape:
            raise ValueError("do must have q's shape and v k's shape")
        if layout == "BHND":
            B, H, Nq, d = q.shape
            Hkv, Nk = k.shape[1], k.shape[2]
            qs = (H * Nq * d, Nq * d, d)
            ks = (Hkv * Nk * d, Nk * d, d)
        elif layout == "BSND":
            B, Nq, H, d = q.shape
            Nk, Hkv = k.shape[1], k.shape[2]
            qs = (Nq * H * d, d, H * d)
            ks = (Nk * Hkv * d, d, Hkv * d)
        else:
            raise ValueError(f"unknown layout {layout!r}")

        def idx(rows, n):
            if rows is None:
                return None, None, n
            a = np.ascontiguousarray(rows, dtype=np.int32)
            return a, a.ctypes.data, int(a.size)

        qa, qp, RQ = idx(qrows, Nq)
        ka, kp, RK = idx(krows, Nk)
        dq = np.empty((B, H, RQ, d), dtype=np.float64) if want_dq else None
        dk = np.empty((B, Hkv, RK, d), dtype=np.float64) if want_dkv else None
        dv = np.empty((B, Hkv, RK, d), dtype=np.float64) if want_dkv else None
        ptr = lambda a: None if a is None else a.ctypes.data
        rc = self._lib.oracle_attn_bwd_ex(
            q.ctypes.data, k.ctypes.data, v.ctypes.data, do.ctypes.data,
            *qs, *ks, B, H, Hkv, Nq, Nk, d, float(scale), int(bool(causal)),
            int(window[0]), int(window[1]), qp, RQ, kp, RK, ptr(dq), ptr(dk), ptr(dv), int(n_threads))
        if rc != 0:
            raise RuntimeError(f"oracle_attn_bwd_ex failed with code {rc}")
        return dq, dk, dv

    def attn_probs(self, q, k, *, scale: float, causal: bool = False):
        """P [Nq, Nk] (float64) of one head; q [Nq,d], k [Nk,d] float32."""
        q = np.ascontiguousarray(q, dtype=np.float32)
        k = np.ascontiguousarray(k, dtype=np.float32)
        Nq, d = q.shape
        Nk = k.shape[0]
        p = np.empty((Nq, Nk), dtype=np.float64)
        rc = self._lib.oracle_attn_probs(q.ctypes.data, k.ctypes.data, d, d,
                                         Nq, Nk, d, float(scale), int(bool(causal)),
                                         p.ctypes.data)
        if rc != 0:
            raise RuntimeError(f"oracle_attn_probs failed with code {rc}")
        return p


_default: OracleLib | None = None


def lib() -> OracleLib:
    """The default oracle library, built on first use if it is missing."""
    global _default
    if _default is None:
        if not os.path.exists(LIBRARY):
            build()
        _default = OracleLib(LIBRARY)
    return _default


def attn_fwd(q, k, v, **kw):
    return lib().attn_fwd(q, k, v, **kw)


def attn_probs(q, k, **kw):
    return lib().attn_probs(q, k, **kw)


def attn_bwd(q, k, v, do, **kw):
    return lib().attn_bwd(q, k, v, do, **kw)


def attn_fwd_ex(q, k, v, **kw):
    return lib().attn_fwd_ex(q, k, v, **kw)


def attn_bwd_ex(q, k, v, do, **kw):
    return lib().attn_bwd_ex(q, k, v, do, **kw)

"""libfa355: attention forward and backward passes on AMD Instinct MI355X
(gfx950).

Python binding of the C ABI in ``include/fa355.h``: argument marshalling only.
Every step of the computation runs in the HIP kernels of ``libfa355.so``;
PyTorch is used for device memory and streams.  There is no CPU fallback:
if the library is not built, or no GPU is present, calls raise.

    O, LSE = fwd(q, k, v, causal=False, scale=None, layout="BHND",
                 out_dtype=torch.float32)

computes O = softmax(scale * Q K^T [causal]) V per (batch, head) and the
per-row natural-log log-sum-exp (pages: [nanhubrain] = nanhubrain.csdn.net
"exact source of the quadratic memory", "tiling skeleton", "online softmax
mathematics"; [ascendai] = ascendai.csdn.net sections 3.1 and 6.1).

    dQ, dK, dV = bwd(q, k, v, o, do, lse, causal=False, scale=None, layout="BHND")

computes the gradients for an upstream gradient dO, rebuilding P from the LSE
([nanhubrain] "backward recomputation"; the row term dO_i . O_i is taken over
the whole row).  Outputs are float32 in the layouts of q and k.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(_PKG, "libfa355.so")

FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_HIP = 0, 1, 2, 3
FA_BHND, FA_BSND = 0, 1
FA_BF16, FA_F32 = 0, 1
LAYOUTS = {"BHND": FA_BHND, "BSND": FA_BSND}

# the symbols include/fa355.h declares
EXPORTS = ("fa_fwd", "fa_fwd_ex", "fa_fwd_sparse", "fa_bwd", "fa_bwd_ex", "fa_bwd_sparse", "fa_decode",
           "fa_decode_workspace_bytes", "fa_decode_noalloc", "fa_status_str",
           "fa_abi_version")
ABI_VERSION = 1

_lib = None


class FaError(RuntimeError):
    """A non-OK fa_status from the library."""

    def __init__(self, status: int, msg: str = ""):
        self.status = status
        super().__init__(f"{fa_status_str(status)}{': ' + msg if msg else ''}")


class FaInvalidArgument(FaError, ValueError):
    pass


class FaUnsupported(FaError, NotImplementedError):
    pass


def load(path: str = LIBRARY) -> ctypes.CDLL:
    """Load libfa355.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it first (python -m exact_attention_112_amd.build "
            "or __graft_entry__.build()); there is no fallback implementation")
    lib = ctypes.CDLL(path)
    lib.fa_fwd.restype = ctypes.c_int
    lib.fa_fwd.argtypes = ([ctypes.c_void_p] * 5 + [ctypes.c_int] * 5 + [ctypes.c_float]
                           + [ctypes.c_int] * 4 + [ctypes.c_void_p])
    lib.fa_fwd_ex.restype = ctypes.c_int
    lib.fa_fwd_ex.argtypes = ([ctypes.c_void_p] * 5 + [ctypes.c_int] * 6 + [ctypes.c_float]
                              + [ctypes.c_int] * 6 + [ctypes.c_void_p])
    lib.fa_fwd_sparse.restype = ctypes.c_int
    lib.fa_fwd_sparse.argtypes = ([ctypes.c_void_p] * 6 + [ctypes.c_int] * 5 + [ctypes.c_float]
                                  + [ctypes.c_int] * 4 + [ctypes.c_void_p])
    lib.fa_decode.restype = ctypes.c_int
    lib.fa_decode.argtypes = ([ctypes.c_void_p] * 8 + [ctypes.c_size_t] + [ctypes.c_int] * 7 + [ctypes.c_float]
                              + [ctypes.c_int] * 3 + [ctypes.c_void_p])
    lib.fa_decode_noalloc.restype = ctypes.c_int
    lib.fa_decode_noalloc.argtypes = ([ctypes.c_void_p] * 7 + [ctypes.c_int] * 7 + [ctypes.c_float]
                                      + [ctypes.c_int] * 3 + [ctypes.c_void_p])
    lib.fa_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.fa_decode_workspace_bytes.argtypes = [ctypes.c_int] * 6
    lib.fa_bwd.restype = ctypes.c_int
    lib.fa_bwd.argtypes = ([ctypes.c_void_p] * 10 + [ctypes.c_int] * 5 + [ctypes.c_float]
                           + [ctypes.c_int] * 4 + [ctypes.c_void_p])
    lib.fa_bwd_ex.restype = ctypes.c_int
    lib.fa_bwd_ex.argtypes = ([ctypes.c_void_p] * 10 + [ctypes.c_int] * 6 + [ctypes.c_float]
                              + [ctypes.c_int] * 6 + [ctypes.c_void_p])
    lib.fa_bwd_sparse.restype = ctypes.c_int
    lib.fa_bwd_sparse.argtypes = ([ctypes.c_void_p] * 11 + [ctypes.c_int] * 5 + [ctypes.c_float]
                                  + [ctypes.c_int] * 4 + [ctypes.c_void_p])
    lib.fa_status_str.restype = ctypes.c_char_p
    lib.fa_status_str.argtypes = [ctypes.c_int]
    lib.fa_abi_version.restype = ctypes.c_int
    lib.fa_abi_version.argtypes = []
    if lib.fa_abi_version() != ABI_VERSION:
        raise ImportError(f"libfa355 ABI {lib.fa_abi_version()} != binding ABI {ABI_VERSION}")
    _lib = lib
    return lib


def fa_status_str(status: int) -> str:
    return load().fa_status_str(int(status)).decode()


def fa_fwd(q: int, k: int, v: int, o: int, lse: int | None, B: int, H: int, Nq: int, Nk: int,
           d: int, scale: float, causal: int, layout: int, in_dtype: int, o_dtype: int,
           stream: int | None) -> int:
    """The C entry point with raw device addresses; returns the fa_status."""
    return int(load().fa_fwd(q, k, v, o, lse or None, B, H, Nq, Nk, d, float(scale),
                             int(causal), int(layout), int(in_dtype), int(o_dtype), stream or None))


def fa_fwd_ex(q: int, k: int, v: int, o: int, lse: int | None, B: int, H: int, Hkv: int, Nq: int, Nk: int,
              d: int, scale: float, causal: int, window_left: int, window_right: int, layout: int,
              in_dtype: int, o_dtype: int, stream: int | None) -> int:
    """The C entry point with raw device addresses; returns the fa_status."""
    return int(load().fa_fwd_ex(q, k, v, o, lse or None, B, H, Hkv, Nq, Nk, d, float(scale), int(causal),
                                int(window_left), int(window_right), int(layout), int(in_dtype),
                                int(o_dtype), stream or None))


def fa_fwd_sparse(q: int, k: int, v: int, o: int, lse: int | None, block_mask: int, B: int, H: int, Nq: int,
                  Nk: int, d: int, scale: float, causal: int, layout: int, in_dtype: int, o_dtype: int,
                  stream: int | None) -> int:
    """The C entry point with raw device addresses; returns the fa_status."""
    return int(load().fa_fwd_sparse(q, k, v, o, lse or None, block_mask, B, H, Nq, Nk, d, float(scale),
                                    int(causal), int(layout), int(in_dtype), int(o_dtype), stream or None))


SPARSE_BQ, SPARSE_BK = 256, 64


def fwd(q, k, v, *, causal: bool = False, scale: float | None = None, layout: str = "BHND",
        out_dtype=None, out=None, lse=None, return_lse: bool = True, window=None, block_mask=None):
    """Attention forward on torch CUDA tensors (ROCm).

    q: [B,H,Nq,d] (BHND) or [B,Nq,H,d] (BSND); k, v: same with Nk and Hkv
    heads, Hkv dividing H (grouped-query attention when Hkv < H).  bf16 or
    fp32, contiguous, on one GPU.  ``window=(left, right)``: key j visible to
    query i iff i-left <= j <= i+right (a negative side is unbounded).
    ``block_mask``: uint8 [B, H, ceil(Nq/256), ceil(Nk/64)] GPU tensor; key
    block j//64 is computed for query block i//256 iff its entry is nonzero.
    Returns (O, LSE): O in q's layout with dtype ``out_dtype`` (default
    float32), LSE float32 [B,H,Nq].  The kernel is enqueued on the current
    stream.
    """
    import torch

    if layout not in LAYOUTS:
        raise ValueError(f"layout must be one of {list(LAYOUTS)}")
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D")
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("q, k, v must be GPU tensors")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on one device")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("q, k, v must share dtype bfloat16 or float32")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous")
    if k.shape != v.shape:
        raise ValueError("k and v must have the same shape")
    if layout == "BHND":
        B, H, Nq, d = q.shape
        Bk, Hk, Nk, dk = k.shape
    else:
        B, Nq, H, d = q.shape
        Bk, Nk, Hk, dk = k.shape
    if Bk != B or dk != d or Hk < 1 or H % Hk != 0:
        raise ValueError(f"q {tuple(q.shape)} and k {tuple(k.shape)} disagree for layout {layout}")
    wl, wr = (-1, -1) if window is None else (int(window[0]), int(window[1]))
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("out_dtype must be float32 or bfloat16")
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    elif out.shape != q.shape or out.dtype != out_dtype or not out.is_contiguous() or out.device != q.device:
        raise ValueError("out must be a contiguous tensor of q's shape, out_dtype and device")
    if return_lse and lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    elif lse is not None and (lse.shape != (B, H, Nq) or lse.dtype != torch.float32
                              or not lse.is_contiguous() or lse.device != q.device):
        raise ValueError("lse must be a contiguous float32 [B,H,Nq] tensor on q's device")
    in_dt = FA_BF16 if q.dtype == torch.bfloat16 else FA_F32
    o_dt = FA_BF16 if out_dtype == torch.bfloat16 else FA_F32
    stream = torch.cuda.current_stream(q.device).cuda_stream
    with torch.cuda.device(q.device):
        sc = -1.0 if scale is None else float(scale)
        lp = lse.data_ptr() if lse is not None else None
        if block_mask is not None:
            nqb, nkb = (Nq + SPARSE_BQ - 1) // SPARSE_BQ, (Nk + SPARSE_BK - 1) // SPARSE_BK
            if (block_mask.shape != (B, H, nqb, nkb) or block_mask.dtype != torch.uint8
                    or not block_mask.is_contiguous() or block_mask.device != q.device):
                raise ValueError(f"block_mask must be a contiguous uint8 [{B},{H},{nqb},{nkb}] tensor on q's device")
            if Hk != H or wl >= 0 or wr >= 0:
                raise ValueError("block_mask does not combine with grouped KV heads or a window")
            st = fa_fwd_sparse(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lp, block_mask.data_ptr(),
                               B, H, Nq, Nk, d, sc, int(bool(causal)), LAYOUTS[layout], in_dt, o_dt, stream)
        elif Hk == H and wl < 0 and wr < 0:
            st = fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lp, B, H, Nq, Nk, d,
                        sc, int(bool(causal)), LAYOUTS[layout], in_dt, o_dt, stream)
        else:
            st = fa_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lp, B, H, Hk, Nq, Nk, d,
                           sc, int(bool(causal)), wl, wr, LAYOUTS[layout], in_dt, o_dt, stream)
    if st == FA_ERR_INVALID_ARG:
        raise FaInvalidArgument(st, "invalid argument")
    if st == FA_ERR_UNSUPPORTED:
        raise FaUnsupported(st, "unsupported configuration")
    if st != FA_OK:
        raise FaError(st, "HIP launch failed")
    return out, lse


def fa_bwd(q: int, k: int, v: int, o: int, dout: int, lse: int, dq: int, dk: int, dv: int, delta: int,
           B: int, H: int, Nq: int, Nk: int, d: int, scale: float, causal: int, layout: int,
           in_dtype: int, o_dtype: int, stream: int | None) -> int:
    """The C entry point with raw device addresses; returns the fa_status."""
    return int(load().fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, Nq, Nk, d, float(scale),
                             int(causal), int(layout), int(in_dtype), int(o_dtype), stream or None))


def fa_bwd_ex(q: int, k: int, v: int, o: int, dout: int, lse: int, dq: int, dk: int, dv: int, delta: int,
              B: int, H: int, Hkv: int, Nq: int, Nk: int, d: int, scale: float, causal: int,
              window_left: int, window_right: int, layout: int, in_dtype: int, o_dtype: int,
              stream: int | None) -> int:
    """The C entry point with raw device addresses; returns the fa_status."""
    return int(load().fa_bwd_ex(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, Hkv, Nq, Nk, d, float(scale),
                                int(causal), int(window_left), int(window_right), int(layout), int(in_dtype),
                                int(o_dtype), stream or None))


def fa_bwd_sparse(q: int, k: int, v: int, o: int, dout: int, lse: int, block_mask: int, dq: int, dk: int,
                  dv: int, delta: int, B: int, H: int, Nq: int, Nk: int, d: int, scale: float, causal: int,
                  layout: int, in_dtype: int, o_dtype: int, stream: int | None) -> int:
    """The C entry point with raw device addresses; returns the fa_status."""
    return int(load().fa_bwd_sparse(q, k, v, o, dout, lse, block_mask, dq, dk, dv, delta, B, H, Nq, Nk, d,
                                    float(scale), int(causal), int(layout), int(in_dtype), int(o_dtype),
                                    stream or None))


def bwd(q, k, v, o, do, lse, *, causal: bool = False, scale: float | None = None, layout: str = "BHND",
        window=None, block_mask=None, dq=None, dk=None, dv=None, delta=None):
    """Attention backward on torch CUDA tensors (ROCm).

    q, k, v, do: bf16, contiguous, in ``layout`` (do has q's shape); o: the
    forward output (float32 or bfloat16, q's shape); lse: float32 [B,H,Nq]
    from the forward pass.  k and v may have fewer heads than q (Hkv dividing
    H: grouped KV heads, as in ``fwd``); ``window`` = (left, right) is the
    band the forward used (None: no band); ``block_mask`` the uint8 [B, H,
    ceil(Nq/256), ceil(Nk/64)] block mask it used (None: dense).  Returns (dQ, dK, dV), float32 in
    the layouts of q and k (dK, dV with k's heads).  ``delta`` (float32
    [B,H,Nq]) is the workspace for D_i; it is allocated here when not given.
    Enqueued on the current stream.
    """
    import torch

    if layout not in LAYOUTS:
        raise ValueError(f"layout must be one of {list(LAYOUTS)}")
    ts = (q, k, v, o, do, lse)
    if any(not t.is_cuda for t in ts) or len({t.device for t in ts}) != 1:
        raise ValueError("all tensors must be on one GPU")
    if not all(t.is_contiguous() for t in ts):
        raise ValueError("all tensors must be contiguous")
    if not (q.dtype == k.dtype == v.dtype == do.dtype == torch.bfloat16):
        raise ValueError("q, k, v and do must be bfloat16")
    if o.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("o must be float32 or bfloat16")
    if q.dim() != 4 or k.shape != v.shape or k.dim() != 4 or do.shape != q.shape or o.shape != q.shape:
        raise ValueError("q, o, do must share a 4-D shape; k and v another")
    if layout == "BHND":
        B, H, Nq, d = q.shape
        Bk, Hk, Nk, dk_ = k.shape
    else:
        B, Nq, H, d = q.shape
        Bk, Nk, Hk, dk_ = k.shape
    if (Bk, dk_) != (B, d) or Hk < 1 or H % Hk != 0:
        raise ValueError(f"q {tuple(q.shape)} and k {tuple(k.shape)} disagree for layout {layout}")
    if lse.shape != (B, H, Nq) or lse.dtype != torch.float32:
        raise ValueError("lse must be float32 [B,H,Nq]")
    wl, wr = (-1, -1) if window is None else (int(window[0]), int(window[1]))

    def out(t, shape, name):
        if t is None:
            return torch.empty(shape, dtype=torch.float32, device=q.device)
        if t.shape != tuple(shape) or t.dtype != torch.float32 or not t.is_contiguous() or t.device != q.device:
            raise ValueError(f"{name} must be a contiguous float32 tensor of shape {tuple(shape)} on q's device")
        return t

    dq = out(dq, q.shape, "dq")
    dk = out(dk, k.shape, "dk")
    dv = out(dv, k.shape, "dv")
    delta = out(delta, (B, H, Nq), "delta")
    o_dt = FA_BF16 if o.dtype == torch.bfloat16 else FA_F32
    stream = torch.cuda.current_stream(q.device).cuda_stream
    with torch.cuda.device(q.device):
        args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(),
                dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr())
        sc = -1.0 if scale is None else float(scale)
        if block_mask is not None:
            nqb, nkb = (Nq + SPARSE_BQ - 1) // SPARSE_BQ, (Nk + SPARSE_BK - 1) // SPARSE_BK
            if (block_mask.dtype != torch.uint8 or tuple(block_mask.shape) != (B, H, nqb, nkb)
                    or not block_mask.is_contiguous() or block_mask.device != q.device):
                raise ValueError(f"block_mask must be a contiguous uint8 tensor of shape {(B, H, nqb, nkb)} "
                                 "on q's device")
            if Hk != H or window is not None:
                raise ValueError("block_mask does not combine with grouped KV heads or a band")
            st = fa_bwd_sparse(*args[:6], block_mask.data_ptr(), *args[6:], B, H, Nq, Nk, d, sc,
                               int(bool(causal)), LAYOUTS[layout], FA_BF16, o_dt, stream)
        elif Hk == H and window is None:
            st = fa_bwd(*args, B, H, Nq, Nk, d, sc, int(bool(causal)), LAYOUTS[layout], FA_BF16, o_dt, stream)
        else:
            st = fa_bwd_ex(*args, B, H, Hk, Nq, Nk, d, sc, int(bool(causal)), wl, wr, LAYOUTS[layout], FA_BF16,
                           o_dt, stream)
    if st == FA_ERR_INVALID_ARG:
        raise FaInvalidArgument(st, "invalid argument")
    if st == FA_ERR_UNSUPPORTED:
        raise FaUnsupported(st, "unsupported configuration")
    if st != FA_OK:
        raise FaError(st, "HIP launch failed")
    return dq, dk, dv


def fa_decode(q: int, k_cache: int, v_cache: int, block_tables: int, seq_lens: int, o: int, lse: int | None,
              workspace: int, workspace_bytes: int, B: int, H: int, Hkv: int, Nq: int, d: int, block_size: int,
              max_blocks: int, scale: float, causal: int, in_dtype: int, o_dtype: int,
              stream: int | None) -> int:
    """The C entry point with raw device addresses; returns the fa_status."""
    return int(load().fa_decode(q, k_cache, v_cache, block_tables, seq_lens, o, lse or None, workspace,
                                int(workspace_bytes), B, H, Hkv, Nq, d, block_size, max_blocks, float(scale),
                                int(causal), int(in_dtype), int(o_dtype), stream or None))


def fa_decode_noalloc(q: int, k_cache: int, v_cache: int, block_tables: int, seq_lens: int, o: int,
                      lse: int | None, B: int, H: int, Hkv: int, Nq: int, d: int, block_size: int, max_blocks: int,
                      scale: float, causal: int, in_dtype: int, o_dtype: int, stream: int | None) -> int:
    """The C entry point without a workspace (the library's fixed device
    array holds the chunk partials); raw device addresses; returns the
    fa_status."""
    return int(load().fa_decode_noalloc(q, k_cache, v_cache, block_tables, seq_lens, o, lse or None, B, H, Hkv,
                                        Nq, d, block_size, max_blocks, float(scale), int(causal), int(in_dtype),
                                        int(o_dtype), stream or None))


# fa_decode_noalloc's limit on the chunk partials (include/fa355.h)
DECODE_NOALLOC_MAX_WORKSPACE = 64 << 20


def fa_decode_workspace_bytes(B: int, H: int, Hkv: int, Nq: int, d: int, max_seq_len: int) -> int:
    return int(load().fa_decode_workspace_bytes(B, H, Hkv, Nq, d, max_seq_len))


def decode(q, k_cache, v_cache, block_tables, seq_lens, *, causal: bool = False, scale: float | None = None,
           out_dtype=None, workspace=None, return_lse: bool = True, out=None, lse=None):
    """Decode attention over a paged KV cache on torch CUDA tensors (ROCm).

    q: [B, Nq, H, d] bf16; k_cache, v_cache: [num_blocks, block_size, Hkv, d]
    bf16; block_tables: int32 [B, max_blocks]; seq_lens: int32 [B].  Returns
    (O [B, Nq, H, d] of ``out_dtype`` (default float32), LSE float32
    [B, H, Nq]).  ``workspace``: optional uint8 device tensor of at least
    fa_decode_workspace_bytes(...) bytes (allocated here when not given).
    """
    import torch

    ts = (q, k_cache, v_cache, block_tables, seq_lens)
    if any(not t.is_cuda for t in ts) or len({t.device for t in ts}) != 1:
        raise ValueError("all tensors must be on one GPU")
    if not all(t.is_contiguous() for t in ts):
        raise ValueError("all tensors must be contiguous")
    if q.dtype != torch.bfloat16 or k_cache.dtype != torch.bfloat16 or v_cache.dtype != torch.bfloat16:
        raise ValueError("q, k_cache, v_cache must be bfloat16")
    if block_tables.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise ValueError("block_tables and seq_lens must be int32")
    if q.dim() != 4 or k_cache.dim() != 4 or k_cache.shape != v_cache.shape:
        raise ValueError("q must be [B,Nq,H,d]; k_cache and v_cache the same [blocks,block_size,Hkv,d]")
    B, Nq, H, d = q.shape
    _, block_size, Hkv, dk = k_cache.shape
    if dk != d or block_tables.dim() != 2 or block_tables.shape[0] != B or seq_lens.shape != (B,):
        raise ValueError("shapes disagree")
    max_blocks = block_tables.shape[1]
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("out_dtype must be float32 or bfloat16")
    need = fa_decode_workspace_bytes(B, H, Hkv, Nq, d, max_blocks * block_size)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    o = torch.empty(q.shape, dtype=out_dtype, device=q.device) if out is None else out
    if o.shape != q.shape or o.dtype != out_dtype or not o.is_contiguous() or o.device != q.device:
        raise ValueError("out must be a contiguous tensor of q's shape and out_dtype on q's device")
    if lse is None and return_lse:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    elif lse is not None and (lse.shape != (B, H, Nq) or lse.dtype != torch.float32 or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous float32 [B,H,Nq] tensor")
    stream = torch.cuda.current_stream(q.device).cuda_stream
    with torch.cuda.device(q.device):
        st = fa_decode(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), block_tables.data_ptr(),
                       seq_lens.data_ptr(), o.data_ptr(), lse.data_ptr() if lse is not None else None,
                       workspace.data_ptr(), workspace.numel() * workspace.element_size(), B, H, Hkv, Nq, d,
                       block_size, max_blocks, -1.0 if scale is None else float(scale), int(bool(causal)),
                       FA_BF16, FA_BF16 if out_dtype == torch.bfloat16 else FA_F32, stream)
    if st == FA_ERR_INVALID_ARG:
        raise FaInvalidArgument(st, "invalid argument")
    if st == FA_ERR_UNSUPPORTED:
        raise FaUnsupported(st, "unsupported configuration")
    if st != FA_OK:
        raise FaError(st, "HIP launch failed")
    return o, lse

"""The C-ABI library without a GPU: it loads, exports every symbol the header
declares, and every argument-validation path returns its status before any HIP
call (so no compute is attempted here)."""
import math
import os
import re
import subprocess

import pytest

import exact_attention_112_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa355.h")


def header_text():
    with open(HEADER) as f:
        return f.read()


def declared_functions():
    return set(re.findall(r"FA355_API\s+[\w\s\*]+?\b(\w+)\s*\(", header_text()))


def test_library_exports_every_declared_symbol():
    lib = fa.load()
    names = declared_functions()
    assert names == set(fa.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", fa.LIBRARY], capture_output=True,
                         text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert names <= exported
    for n in names:
        assert hasattr(lib, n)
    # nothing else leaks out of the library as a function symbol
    assert exported == names


def test_header_constants_match_binding():
    t = header_text()
    consts = {k: int(v) for k, v in re.findall(r"\b(FA_[A-Z0-9_]+)\s*=\s*(\d+)", t)}
    for name, val in consts.items():
        assert getattr(fa, name) == val, name
    assert int(re.search(r"#define FA355_ABI_VERSION (\d+)", t).group(1)) == fa.ABI_VERSION
    assert fa.load().fa_abi_version() == fa.ABI_VERSION


def test_status_strings():
    assert fa.fa_status_str(0) == "FA_OK"
    assert fa.fa_status_str(1) == "FA_ERR_INVALID_ARG"
    assert fa.fa_status_str(2) == "FA_ERR_UNSUPPORTED"
    assert fa.fa_status_str(3) == "FA_ERR_HIP"
    assert fa.fa_status_str(99) == "FA_UNKNOWN_STATUS"


# Fake, 16-byte-aligned, never-dereferenced addresses: validation rejects every
# case below before anything would touch them.
P = 0x10000
GOOD = dict(q=P, k=P + 0x1000, v=P + 0x2000, o=P + 0x3000, lse=P + 0x4000, B=1, H=2, Nq=16,
            Nk=16, d=64, scale=-1.0, causal=0, layout=fa.FA_BHND, in_dtype=fa.FA_BF16,
            o_dtype=fa.FA_F32, stream=None)


def call(**changes):
    a = dict(GOOD, **changes)
    return fa.fa_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Nq"], a["Nk"],
                     a["d"], a["scale"], a["causal"], a["layout"], a["in_dtype"], a["o_dtype"],
                     a["stream"])


@pytest.mark.parametrize("changes,status", [
    (dict(q=0), fa.FA_ERR_INVALID_ARG),
    (dict(k=0), fa.FA_ERR_INVALID_ARG),
    (dict(v=0), fa.FA_ERR_INVALID_ARG),
    (dict(o=0), fa.FA_ERR_INVALID_ARG),
    (dict(B=0), fa.FA_ERR_INVALID_ARG),
    (dict(H=-1), fa.FA_ERR_INVALID_ARG),
    (dict(Nq=0), fa.FA_ERR_INVALID_ARG),
    (dict(Nk=0), fa.FA_ERR_INVALID_ARG),
    (dict(d=0), fa.FA_ERR_INVALID_ARG),
    (dict(layout=2), fa.FA_ERR_INVALID_ARG),
    (dict(in_dtype=7), fa.FA_ERR_INVALID_ARG),
    (dict(o_dtype=-1), fa.FA_ERR_INVALID_ARG),
    (dict(q=P + 8), fa.FA_ERR_INVALID_ARG),          # misaligned
    (dict(o=P + 0x3004), fa.FA_ERR_INVALID_ARG),
    (dict(lse=P + 0x4002), fa.FA_ERR_INVALID_ARG),
    (dict(scale=math.nan), fa.FA_ERR_INVALID_ARG),
    (dict(scale=math.inf), fa.FA_ERR_INVALID_ARG),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(d=256), fa.FA_ERR_UNSUPPORTED),
    (dict(in_dtype=fa.FA_F32, o_dtype=fa.FA_BF16), fa.FA_ERR_UNSUPPORTED),
    (dict(B=1 << 16, H=1 << 16), fa.FA_ERR_UNSUPPORTED),   # grid beyond 2^31 workgroups
])
def test_validation_returns_before_launch(changes, status):
    assert call(**changes) == status


def test_python_wrapper_validates_without_gpu():
    import torch
    x = torch.zeros(1, 1, 4, 64)
    with pytest.raises(ValueError):
        fa.fwd(x, x, x)                        # CPU tensors are refused
    with pytest.raises(ValueError):
        fa.fwd(x, x, x, layout="NHWC")


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(ImportError):
        fa.load.__wrapped__(str(tmp_path / "nope.so")) if hasattr(fa.load, "__wrapped__") else \
            _load_fresh(str(tmp_path / "nope.so"))


def _load_fresh(path):
    saved = fa._lib
    fa._lib = None
    try:
        fa.load(path)
    finally:
        fa._lib = saved


BGOOD = dict(q=P, k=P + 0x1000, v=P + 0x2000, o=P + 0x3000, do=P + 0x5000, lse=P + 0x4000,
             dq=P + 0x6000, dk=P + 0x7000, dv=P + 0x8000, delta=P + 0x9000, B=1, H=2, Nq=16, Nk=16,
             d=64, scale=-1.0, causal=0, layout=fa.FA_BHND, in_dtype=fa.FA_BF16, o_dtype=fa.FA_F32,
             stream=None)


def bcall(**changes):
    a = dict(BGOOD, **changes)
    return fa.fa_bwd(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"], a["dk"], a["dv"],
                     a["delta"], a["B"], a["H"], a["Nq"], a["Nk"], a["d"], a["scale"], a["causal"],
                     a["layout"], a["in_dtype"], a["o_dtype"], a["stream"])


@pytest.mark.parametrize("changes,status", [
    *[(dict(**{name: 0}), fa.FA_ERR_INVALID_ARG)
      for name in ("q", "k", "v", "o", "do", "lse", "dq", "dk", "dv", "delta")],
    (dict(B=0), fa.FA_ERR_INVALID_ARG),
    (dict(Nq=-3), fa.FA_ERR_INVALID_ARG),
    (dict(Nk=0), fa.FA_ERR_INVALID_ARG),
    (dict(layout=5), fa.FA_ERR_INVALID_ARG),
    (dict(in_dtype=3), fa.FA_ERR_INVALID_ARG),
    (dict(o_dtype=9), fa.FA_ERR_INVALID_ARG),
    (dict(do=P + 0x5008), fa.FA_ERR_INVALID_ARG),    # misaligned
    (dict(dk=P + 0x7004), fa.FA_ERR_INVALID_ARG),
    (dict(delta=P + 0x9002), fa.FA_ERR_INVALID_ARG),
    (dict(scale=math.nan), fa.FA_ERR_INVALID_ARG),
    (dict(scale=-math.inf), fa.FA_ERR_INVALID_ARG),
    (dict(d=32), fa.FA_ERR_UNSUPPORTED),
    (dict(in_dtype=fa.FA_F32), fa.FA_ERR_UNSUPPORTED),
    (dict(B=1 << 16, H=1 << 16), fa.FA_ERR_UNSUPPORTED),
])
def test_bwd_validation_returns_before_launch(changes, status):
    assert bcall(**changes) == status


BXGOOD = dict(BGOOD, H=4, Hkv=2, wl=8, wr=-1)


def bxcall(**changes):
    a = dict(BXGOOD, **changes)
    return fa.fa_bwd_ex(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"], a["dk"], a["dv"],
                        a["delta"], a["B"], a["H"], a["Hkv"], a["Nq"], a["Nk"], a["d"], a["scale"], a["causal"],
                        a["wl"], a["wr"], a["layout"], a["in_dtype"], a["o_dtype"], a["stream"])


@pytest.mark.parametrize("changes,status", [
    (dict(dv=0), fa.FA_ERR_INVALID_ARG),
    (dict(Hkv=0), fa.FA_ERR_INVALID_ARG),
    (dict(H=6, Hkv=4), fa.FA_ERR_INVALID_ARG),      # H not a multiple of Hkv
    (dict(Nk=0), fa.FA_ERR_INVALID_ARG),
    (dict(layout=2), fa.FA_ERR_INVALID_ARG),
    (dict(dq=P + 0x6004), fa.FA_ERR_INVALID_ARG),
    (dict(scale=math.inf), fa.FA_ERR_INVALID_ARG),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(in_dtype=fa.FA_F32), fa.FA_ERR_UNSUPPORTED),
    (dict(Nq=1 << 30), fa.FA_ERR_UNSUPPORTED),
])
def test_bwd_ex_validation_returns_before_launch(changes, status):
    assert bxcall(**changes) == status


def bscall(**changes):
    a = dict(dict(BGOOD, mask=P + 0xa000), **changes)
    return fa.fa_bwd_sparse(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["mask"], a["dq"], a["dk"],
                            a["dv"], a["delta"], a["B"], a["H"], a["Nq"], a["Nk"], a["d"], a["scale"], a["causal"],
                            a["layout"], a["in_dtype"], a["o_dtype"], a["stream"])


@pytest.mark.parametrize("changes,status", [
    (dict(mask=0), fa.FA_ERR_INVALID_ARG),           # the mask is required
    (dict(dq=0), fa.FA_ERR_INVALID_ARG),
    (dict(Nq=0), fa.FA_ERR_INVALID_ARG),
    (dict(lse=P + 0x4002), fa.FA_ERR_INVALID_ARG),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(Nk=64 * 4096 + 1), fa.FA_ERR_UNSUPPORTED),   # more key blocks than a list holds
    (dict(Nq=256 * 4096 + 1), fa.FA_ERR_UNSUPPORTED),  # more query blocks than a list holds
])
def test_bwd_sparse_validation_returns_before_launch(changes, status):
    assert bscall(**changes) == status


def test_bwd_python_wrapper_validates_without_gpu():
    import torch
    x = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    l = torch.zeros(1, 1, 4)
    with pytest.raises(ValueError):
        fa.bwd(x, x, x, x, x, l)               # CPU tensors are refused


XGOOD = dict(GOOD, Hkv=2, wl=-1, wr=-1)


def xcall(**changes):
    a = dict(XGOOD, **changes)
    return fa.fa_fwd_ex(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Hkv"], a["Nq"], a["Nk"],
                        a["d"], a["scale"], a["causal"], a["wl"], a["wr"], a["layout"], a["in_dtype"],
                        a["o_dtype"], a["stream"])


@pytest.mark.parametrize("changes,status", [
    (dict(q=0), fa.FA_ERR_INVALID_ARG),
    (dict(Hkv=0), fa.FA_ERR_INVALID_ARG),
    (dict(H=3, Hkv=2), fa.FA_ERR_INVALID_ARG),      # H not a multiple of Hkv
    (dict(Nk=0), fa.FA_ERR_INVALID_ARG),
    (dict(layout=3), fa.FA_ERR_INVALID_ARG),
    (dict(v=P + 0x2004), fa.FA_ERR_INVALID_ARG),
    (dict(scale=math.nan), fa.FA_ERR_INVALID_ARG),
    (dict(d=80), fa.FA_ERR_UNSUPPORTED),
    (dict(in_dtype=fa.FA_F32, H=2, Hkv=1), fa.FA_ERR_UNSUPPORTED),   # fp32: plain attention only
    (dict(in_dtype=fa.FA_F32, wl=4), fa.FA_ERR_UNSUPPORTED),
    (dict(Nq=1 << 30), fa.FA_ERR_UNSUPPORTED),
    (dict(Nk=1 << 30), fa.FA_ERR_UNSUPPORTED),
])
def test_fwd_ex_validation_returns_before_launch(changes, status):
    assert xcall(**changes) == status


DGOOD = dict(q=P, kc=P + 0x1000, vc=P + 0x2000, bt=P + 0x3000, sl=P + 0x4000, o=P + 0x5000, lse=P + 0x6000,
             ws=P + 0x7000, ws_bytes=1 << 30, B=2, H=4, Hkv=2, Nq=1, d=128, bs=16, mb=8, scale=-1.0, causal=0,
             in_dtype=fa.FA_BF16, o_dtype=fa.FA_F32, stream=None)


def dcall(**changes):
    a = dict(DGOOD, **changes)
    return fa.fa_decode(a["q"], a["kc"], a["vc"], a["bt"], a["sl"], a["o"], a["lse"], a["ws"], a["ws_bytes"],
                        a["B"], a["H"], a["Hkv"], a["Nq"], a["d"], a["bs"], a["mb"], a["scale"], a["causal"],
                        a["in_dtype"], a["o_dtype"], a["stream"])


@pytest.mark.parametrize("changes,status", [
    *[(dict(**{name: 0}), fa.FA_ERR_INVALID_ARG) for name in ("q", "kc", "vc", "bt", "sl", "o", "ws")],
    (dict(B=0), fa.FA_ERR_INVALID_ARG),
    (dict(H=6, Hkv=4), fa.FA_ERR_INVALID_ARG),
    (dict(bs=24), fa.FA_ERR_INVALID_ARG),          # not a power of two
    (dict(bs=8), fa.FA_ERR_INVALID_ARG),           # below 16
    (dict(mb=0), fa.FA_ERR_INVALID_ARG),
    (dict(bt=P + 0x3002), fa.FA_ERR_INVALID_ARG),
    (dict(ws=P + 0x7008), fa.FA_ERR_INVALID_ARG),
    (dict(ws_bytes=16), fa.FA_ERR_INVALID_ARG),    # workspace too small
    (dict(scale=math.inf), fa.FA_ERR_INVALID_ARG),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(in_dtype=fa.FA_F32), fa.FA_ERR_UNSUPPORTED),
])
def test_decode_validation_returns_before_launch(changes, status):
    assert dcall(**changes) == status


def test_decode_workspace_formula():
    # B*H*Nq*S*(d+1) floats with S = min(ceil(2048 / (B*Hkv*row tiles)), ceil(max_len / 256))
    assert fa.fa_decode_workspace_bytes(2, 4, 2, 1, 128, 128) == 2 * 4 * 1 * 1 * 129 * 4
    assert fa.fa_decode_workspace_bytes(2, 4, 2, 1, 128, 100000) == 2 * 4 * 1 * 391 * 129 * 4
    assert fa.fa_decode_workspace_bytes(32, 32, 8, 1, 128, 8192) == 32 * 32 * 8 * 129 * 4
    assert fa.fa_decode_workspace_bytes(0, 4, 2, 1, 128, 128) == 0


SGOOD = dict(GOOD, mask=P + 0x9000)


def scall(**changes):
    a = dict(SGOOD, **changes)
    return fa.fa_fwd_sparse(a["q"], a["k"], a["v"], a["o"], a["lse"], a["mask"], a["B"], a["H"], a["Nq"],
                            a["Nk"], a["d"], a["scale"], a["causal"], a["layout"], a["in_dtype"], a["o_dtype"],
                            a["stream"])


@pytest.mark.parametrize("changes,status", [
    (dict(mask=0), fa.FA_ERR_INVALID_ARG),
    (dict(q=0), fa.FA_ERR_INVALID_ARG),
    (dict(Nk=0), fa.FA_ERR_INVALID_ARG),
    (dict(d=32), fa.FA_ERR_UNSUPPORTED),
    (dict(in_dtype=fa.FA_F32), fa.FA_ERR_UNSUPPORTED),
    (dict(Nk=64 * 4096 + 1), fa.FA_ERR_UNSUPPORTED),   # more key blocks than the tile list holds
])
def test_fwd_sparse_validation_returns_before_launch(changes, status):
    assert scall(**changes) == status


def test_sparse_granularity_matches_header():
    t = header_text()
    assert int(re.search(r"#define FA_SPARSE_BQ (\d+)", t).group(1)) == fa.SPARSE_BQ
    assert int(re.search(r"#define FA_SPARSE_BK (\d+)", t).group(1)) == fa.SPARSE_BK

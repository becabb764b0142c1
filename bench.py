"""Benchmark of the attention forward pass (default) or backward pass on one
MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--pass fwd|bwd]

One step = one call of the HIP forward kernel (the whole hot path: Q tile
load, K/V staging, S = Q K^T, mask, online softmax, P V, epilogue) over the
workload's batch, inputs resident in HBM.  Prints one JSON line with the
throughput in TFLOP/s (4*B*H*Nq*Nk*d, halved for causal) and:

* roofline: the kernel's achieved TFLOP/s against MI355X's dense bf16 MFMA peak
  (2.5 PFLOP/s), timed live with HIP events on the stream the kernel runs on;
  ``traffic`` is the HBM bytes per launch from the committed rocprofv3 counter
  summary, or null when the kernel source changed since it was taken;
* latency_ms: mean, median, min and max of the per-launch times (a second
  pass of as many launches, with a HIP event between consecutive launches),
  and the TFLOP/s at the median;
* counters: the matrix-core busy fraction, vector-ALU busy fraction, LDS bank
  conflicts and HBM rate from the committed rocprofv3 counter summary of the
  current kernel source (null otherwise);
* cpu_baseline: the fp64 CPU oracle timed on this host's cores on a bounded
  sample of the same workload (rows of the first heads, about 10 s of work),
  with the host's CPU model and core counts and the extrapolated time of a
  full oracle run, as a reported baseline, not a target;
* context: the pages' own latency figures with their hardware (Ascend 910B,
  Atlas 800), for context only.

``--workload all`` runs the five forward workloads one after another (30
timed launches after 5 warmup launches and at least one second of warmup;
10 after 2 for the 128K context), prints one line each and, with ``--out
PATH``, writes them to a JSON file.

With ``--pass bwd`` one step is one fa_bwd call (D = rowsum(dO*O), the dK/dV
kernel and the dQ kernel) on the workload, given O and LSE from one forward
call made before the timed region; the throughput counts the backward's five
products, 2.5x the forward's flops (10*B*H*Nq*Nk*d, halved for causal), and
the roofline is that of the whole call.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOPS and % of bf16 MFMA peak at B4 H32 N8192 d128"
BWD_METRIC = "attention bwd TFLOPS and % of bf16 MFMA peak at B4 H32 N8192 d128"
PEAK_BF16_TFLOPS = 2500.0          # MI355X dense bf16 MFMA (published)
PEAK_F32_TFLOPS = 157.3            # MI355X fp32 (matrix and vector), published
PEAK_HBM_GBS = 8000.0              # MI355X HBM3E
# the five forward workloads (tiny fp32, causal prefill, the headline
# self-attention, cross-attention on 77 keys, the 128K causal context)
FORWARD_WORKLOADS = ["tiny_f32", "llama_prefill_causal", "selfattn_b4h32n8k", "sd_crossattn", "long_causal_128k"]


def bwd_algorithmic_bytes(w) -> float:
    """Read Q, K, V, dO (bf16), O (fp32) and LSE once; write dQ, dK, dV (fp32) once
    (K, V, dK and dV have w.kv_heads heads)."""
    q_side = w.H * (2 * w.Nq * w.d * 2 + w.Nq * w.d * 4 + w.Nq * 4 + w.Nq * w.d * 4)
    kv_side = w.kv_heads * (2 * w.Nk * w.d * 2 + 2 * w.Nk * w.d * 4)
    return float(q_side + kv_side) * w.B


def algorithmic_bytes(w, out_bytes: int) -> float:
    """Read Q, K, V once (K and V have w.kv_heads heads), write O and LSE once (per launch)."""
    el = 2 if w.dtype == "bf16" else 4
    q_side = w.H * (w.Nq * w.d * el + w.Nq * w.d * out_bytes + w.Nq * 4)
    kv_side = w.kv_heads * 2 * w.Nk * w.d * el
    return float(q_side + kv_side) * w.B


# the kernels' sources (their file and the shared device header)
KERNEL_SOURCES = {
    p: [os.path.join(ROOT, "exact_attention_112_amd", "csrc", n) for n in (f"fa_{p}.hip", "fa_common.h")]
    for p in ("fwd", "bwd", "decode")
}
PROFILES = os.path.join(ROOT, "profiles")


def kernel_source_hash(which: str = "fwd") -> str:
    h = hashlib.sha256()
    for path in KERNEL_SOURCES[which]:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(workload: str, which: str = "fwd"):
    """HBM bytes per launch from profiles/fa_<which>_<workload>_counters.md, if
    the summary was taken on the current kernel source; else None."""
    path = os.path.join(PROFILES, f"fa_{which}_{workload}_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != kernel_source_hash(which):
        return None
    return float(m_bytes.group(1))


def counters_from_profiles(workload: str, which: str = "fwd"):
    """The SQ counter figures (matrix-core busy, vector-ALU busy, LDS bank
    conflicts, HBM rate) recorded in profiles/fa_<which>_<workload>_counters.md
    for the current kernel source, or None."""
    path = os.path.join(PROFILES, f"fa_{which}_{workload}_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    if not m_hash or m_hash.group(1) != kernel_source_hash(which):
        return None
    out = {}
    for key in ("mfma_busy_frac", "valu_busy_frac", "lds_bank_conflict_frac", "hbm_gbs", "clock_ghz"):
        m = re.search(rf"{key}:\s*([0-9.eE+-]+)", text)
        if m:
            out[key] = float(m.group(1))
    return out or None


def host_cpu():
    """The host's CPU model and core counts (for the CPU baseline's record)."""
    model, cores = None, set()
    try:
        phys = core = None
        for line in open("/proc/cpuinfo"):
            key, _, val = line.partition(":")
            key, val = key.strip(), val.strip()
            if key == "model name" and model is None:
                model = val
            elif key == "physical id":
                phys = val
            elif key == "core id":
                core = val
                cores.add((phys, core))
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count()
    return {"cpu_model": model, "physical_cores": len(cores) or None, "logical_cpus": os.cpu_count(),
            "usable_cpus": usable, "omp_num_threads": os.environ.get("OMP_NUM_THREADS")}


# The pages' own latency figures for this path, with their hardware: other
# machines, precision and masking not stated, so context only (not a target).
PAGES_CONTEXT = [
    {"source": "[pwwt] www.pwwt.cn/news/2518640, section on measured performance",
     "hardware": "Huawei Ascend 910B", "workload": "LLaMA-13B inference (batch and masking not stated)",
     "seq_len": [2048, 4096, 8192], "flash_attention_ms": [18, 38, 82], "standard_attention_ms": [42, 156, "OOM"]},
    {"source": "[ascendai] ascendai.csdn.net, section 4.3 (performance comparison)",
     "hardware": "Huawei Atlas 800", "workload": "B=4 H=32 D=128 (masking not stated)",
     "seq_len": [2048, 8192, 32768, 131072], "flash_attention_ms": [6.2, 24, 95, 380],
     "standard_attention_ms": [8.5, 125, "OOM", "OOM"]},
]


def cpu_baseline(w, inp, target_s: float = 10.0):
    """Time the fp64 oracle on every 4th query row (every Nq/2048-th on longer
    sequences) of consecutive heads until at least ``target_s`` seconds of
    work are done (bounded by the workload); also extrapolates the time of a
    full oracle run by the flop ratio (an estimate)."""
    import numpy as np
    import oracle

    lib = oracle.lib()
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or lib.max_threads()
    stride = max(4, w.Nq // 2048)                # at most 2048 rows of a head
    rows = np.arange(0, w.Nq, stride, dtype=np.int32)
    heads_per_chunk = 2
    done_heads, flops, elapsed = 0, 0.0, 0.0
    total_heads = w.B * w.H
    extended = w.kv_heads != w.H or w.window != (-1, -1)
    group = w.H // w.kv_heads

    def n_visible(i):
        lo = max(0, i - w.window[0]) if w.window[0] >= 0 else 0
        hi = min(w.Nk - 1, i + w.window[1]) if w.window[1] >= 0 else w.Nk - 1
        if w.causal:
            hi = min(hi, i)
        return max(0, hi - lo + 1)

    per_head = float(sum(4.0 * n_visible(int(r)) * w.d for r in rows))
    while done_heads < total_heads and elapsed < target_s:
        n = min(heads_per_chunk, total_heads - done_heads)
        sl = []
        for t in range(done_heads, done_heads + n):
            b, h = divmod(t, w.H)
            hk = h // group
            if w.layout == "BHND":
                sl.append((inp.q[b:b + 1, h:h + 1], inp.k[b:b + 1, hk:hk + 1], inp.v[b:b + 1, hk:hk + 1]))
            else:
                sl.append((inp.q[b:b + 1, :, h:h + 1], inp.k[b:b + 1, :, hk:hk + 1], inp.v[b:b + 1, :, hk:hk + 1]))
        t0 = time.perf_counter()
        for q, k, v in sl:
            if extended:
                lib.attn_fwd_ex(q, k, v, scale=w.scale, causal=w.causal, window=w.window, layout=w.layout,
                                rows=rows, n_threads=threads)
            else:
                lib.attn_fwd(q, k, v, scale=w.scale, causal=w.causal, layout=w.layout, rows=rows,
                             n_threads=threads)
        elapsed += time.perf_counter() - t0
        flops += n * per_head
        done_heads += n
    return {
        "value": flops / elapsed / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"fp64 two-pass oracle on every {stride}th query row ({len(rows)} rows) of the first "
                   f"{done_heads} of {total_heads} heads of {w.name}; {flops:.3e} flop in "
                   f"{elapsed:.1f} s on {threads} threads"),
        "host": host_cpu(),
        "full_run_s_estimate": round(w.flops / (flops / elapsed), 1),
    }


def cpu_baseline_bwd(w, inp, grad, target_s: float = 10.0):
    """Time the fp64 backward oracle head by head (in (b, h) order; with grouped
    KV heads, one KV head's group of query heads at a time) until at least
    ``target_s`` seconds of work are done: per head, the row statistics of the
    queries the outputs need plus dQ of every 4th query row and dK, dV of every
    4th key row.  The rate counts the algorithmic backward flops of the rows
    returned (dQ is 2 of the backward's 5 products, dK and dV 3 of them)."""
    import numpy as np
    import oracle

    lib = oracle.lib()
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or lib.max_threads()
    qrows = np.arange(0, w.Nq, 4, dtype=np.int32)
    krows = np.arange(0, w.Nk, 4, dtype=np.int32)
    per_head = 2.5 * w.flops / (w.B * w.H)
    frac = 0.4 * len(qrows) / w.Nq + 0.6 * len(krows) / w.Nk
    extended = w.kv_heads != w.H or w.window != (-1, -1)
    group = w.H // w.kv_heads
    done, elapsed = 0, 0.0
    while done < w.B * w.H and elapsed < target_s:
        b, h = divmod(done, w.H)
        n = group if extended else 1                 # query heads in this call
        hk = h // group
        if w.layout == "BHND":
            sq = lambda x: x[b:b + 1, h:h + n]
            sk = lambda x: x[b:b + 1, hk:hk + 1] if extended else x[b:b + 1, h:h + 1]
        else:
            sq = lambda x: x[b:b + 1, :, h:h + n]
            sk = lambda x: x[b:b + 1, :, hk:hk + 1] if extended else x[b:b + 1, :, h:h + 1]
        t0 = time.perf_counter()
        if extended:
            lib.attn_bwd_ex(sq(inp.q), sk(inp.k), sk(inp.v), sq(grad), scale=w.scale, causal=w.causal,
                            window=w.window, layout=w.layout, qrows=qrows, krows=krows, n_threads=threads)
        else:
            lib.attn_bwd(sq(inp.q), sk(inp.k), sk(inp.v), sq(grad), scale=w.scale, causal=w.causal,
                         layout=w.layout, qrows=qrows, krows=krows, n_threads=threads)
        elapsed += time.perf_counter() - t0
        done += n
    flops = done * per_head * frac
    return {
        "value": flops / elapsed / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"fp64 backward oracle on the first {done} of {w.B * w.H} heads of {w.name}: row "
                   f"statistics of the queries the outputs need, dQ of every 4th query row, dK and dV of "
                   f"every 4th key row; {flops:.3e} algorithmic flop in {elapsed:.1f} s on {threads} threads"),
    }


def sparse_pair_flops(w, mask) -> float:
    """4*d per (query, key) pair the block mask lets through (no causal here)."""
    import numpy as np
    rows = np.minimum(256, w.Nq - 256 * np.arange(mask.shape[2]))
    cols = np.minimum(64, w.Nk - 64 * np.arange(mask.shape[3]))
    pairs = float(np.einsum("bhqk,q,k->", mask.astype(np.float64), rows.astype(np.float64),
                            cols.astype(np.float64)))
    return 4.0 * w.d * pairs


def cpu_baseline_sparse(w, inp, mask, target_s: float = 10.0):
    """Time the block-sparse oracle (numpy fp64) on every 16th query row of
    consecutive heads until ``target_s`` seconds are done."""
    import numpy as np
    from oracle import sparse

    rows = np.arange(0, w.Nq, 16)
    done, elapsed, flops = 0, 0.0, 0.0
    bh = (lambda x: x) if w.layout == "BHND" else (lambda x: x.transpose(0, 2, 1, 3))
    Q, K, V = bh(inp.q), bh(inp.k), bh(inp.v)
    while done < w.B * w.H and elapsed < target_s:
        b, h = divmod(done, w.H)
        t0 = time.perf_counter()
        sparse.attn_fwd_block_sparse(Q[b, h], K[b, h], V[b, h], mask[b, h], bq=256, bk=64, scale=w.scale,
                                     causal=w.causal, rows=rows)
        elapsed += time.perf_counter() - t0
        cols = np.minimum(64, w.Nk - 64 * np.arange(mask.shape[3]))
        flops += 4.0 * w.d * float(sum((mask[b, h, r // 256] * cols).sum() for r in rows))
        done += 1
    return {
        "value": flops / elapsed / 1e12,
        "unit": "TFLOP/s",
        "cores": 1,
        "kind": "oracle",
        "sample": (f"numpy fp64 block-sparse oracle on every 16th query row of the first {done} of {w.B * w.H} "
                   f"heads of {w.name}; {flops:.3e} flop in {elapsed:.1f} s"),
    }


def cpu_baseline_bwd_sparse(w, inp, grad, mask, target_s: float = 10.0):
    """Time the block-sparse backward oracle (numpy fp64) head by head until
    ``target_s`` seconds are done: per head, the row statistics of every
    query plus dQ of every 16th query row and dK, dV of every 16th key row.
    The rate counts the algorithmic backward flops of the rows returned (2.5 x
    the forward's per visible pair; dQ is 2 of the 5 products, dK and dV 3)."""
    import numpy as np
    from oracle import sparse
    try:
        from threadpoolctl import threadpool_info
        threads = max([int(i.get("num_threads", 1)) for i in threadpool_info() if i.get("user_api") == "blas"]
                      or [1])
    except Exception:   # noqa: BLE001 (the count is informational)
        threads = 1
    qrows = np.arange(0, w.Nq, 16)
    krows = np.arange(0, w.Nk, 16)
    bh = (lambda x: x) if w.layout == "BHND" else (lambda x: x.transpose(0, 2, 1, 3))
    Q, K, V, G = bh(inp.q), bh(inp.k), bh(inp.v), bh(grad)
    cols = np.minimum(64, w.Nk - 64 * np.arange(mask.shape[3]))
    done, elapsed, flops = 0, 0.0, 0.0
    while done < w.B * w.H and elapsed < target_s:
        b, h = divmod(done, w.H)
        t0 = time.perf_counter()
        sparse.attn_bwd_block_sparse(Q[b, h], K[b, h], V[b, h], G[b, h], mask[b, h], bq=256, bk=64,
                                     scale=w.scale, causal=w.causal, qrows=qrows, krows=krows)
        elapsed += time.perf_counter() - t0
        pairs = float((mask[b, h] * cols[None, :]).sum(axis=1) @ np.minimum(256, w.Nq - 256 * np.arange(mask.shape[2])))
        flops += 2.5 * 4.0 * w.d * pairs * (0.4 * len(qrows) / w.Nq + 0.6 * len(krows) / w.Nk)
        done += 1
    return {
        "value": flops / elapsed / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"numpy fp64 block-sparse backward oracle on the first {done} of {w.B * w.H} heads of "
                   f"{w.name}: row statistics of every query, dQ of every 16th query row, dK and dV of every "
                   f"16th key row; {flops:.3e} algorithmic flop in {elapsed:.1f} s"),
    }


def decode_bytes(w, lens) -> float:
    """Algorithmic bytes of one decode call: every cached K and V row of every
    sequence read once (bf16), Q read and O (fp32) and LSE written once, the
    block tables and lengths read once."""
    kv = 2.0 * float(sum(int(x) for x in lens)) * w.Hkv * w.d * 2
    qo = w.B * w.Nq * w.H * w.d * (2 + 4) + w.B * w.H * w.Nq * 4
    return kv + qo + w.B * w.max_blocks * 4 + w.B * 4


def cpu_baseline_decode(w, inp, target_s: float = 10.0):
    """Time the decode oracle (block-table gather + fp64 forward) sequence by
    sequence until ``target_s`` seconds are done; rate in GB/s of the
    algorithmic bytes of the sequences covered."""
    import oracle
    from oracle import paged

    lib = oracle.lib()
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or lib.max_threads()
    done, elapsed, nbytes = 0, 0.0, 0.0
    while done < w.B and elapsed < target_s:
        b = done
        t0 = time.perf_counter()
        paged.decode_reference(lib, inp.q[b:b + 1], inp.k_cache, inp.v_cache, inp.block_tables[b:b + 1],
                               inp.seq_lens[b:b + 1], scale=w.scale, causal=w.causal)
        elapsed += time.perf_counter() - t0
        nbytes += decode_bytes(w.scaled(B=1), inp.seq_lens[b:b + 1])
        done += 1
    return {
        "value": nbytes / elapsed / 1e9,
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"block-table gather + fp64 oracle on the first {done} of {w.B} sequences of {w.name}; "
                   f"{nbytes:.3e} algorithmic bytes in {elapsed:.1f} s on {threads} threads"),
    }


def bench_decode(args, w):
    """One step = one fa_decode call (split kernel + merge kernel)."""
    import numpy as np
    import torch
    import exact_attention_112_amd as fa
    from exact_attention_112_amd import inputs as I

    print(f"bench: generating inputs for {w.name}", file=sys.stderr, flush=True)
    inp = I.make_paged(w)
    t = lambda bits: torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to("cuda")
    tq, kc, vc = t(inp.q_bits), t(inp.k_bits), t(inp.v_bits)
    bt = torch.from_numpy(inp.block_tables).to("cuda")
    sl = torch.from_numpy(inp.seq_lens).to("cuda")
    need = fa.fa_decode_workspace_bytes(w.B, w.H, w.Hkv, w.Nq, w.d, w.max_blocks * w.block_size)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    o = torch.empty(tq.shape, dtype=torch.float32, device="cuda")
    lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device="cuda")

    def step():
        fa.decode(tq, kc, vc, bt, sl, causal=w.causal, scale=w.scale, workspace=ws, out=o, lse=lse)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    if not torch.isfinite(o).all():
        print("bench: non-finite output", file=sys.stderr)
        return 1
    nbytes = decode_bytes(w, inp.seq_lens)
    gbs = nbytes / (ms * 1e-3) / 1e9
    cpu = None if args.no_cpu_baseline else cpu_baseline_decode(w, inp)
    line = {
        "metric": f"attention decode GB/s and % of HBM peak at {w.name}",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) Q and paged K/V cache, seeded lengths and block placement)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "Hkv": w.Hkv, "Nq": w.Nq, "max_len": w.max_len,
                   "min_len": w.min_len, "d": w.d, "block_size": w.block_size, "causal": w.causal,
                   "pass": "decode"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4),
                     "traffic": traffic_from_profiles(w.name, "decode")},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


def bench_attention(args, w, steps: int, warmup: int, with_cpu: bool, min_warmup_s: float = 0.0):
    """Time ``steps`` calls of the forward (or, with args.which == "bwd", the
    backward) pass on workload ``w`` after ``warmup`` untimed calls; returns
    the JSON record (None on a non-finite output).  With ``min_warmup_s`` the
    warmup continues past ``warmup`` calls until that much time has passed
    (short kernels: the GPU clock ramps up over tens of milliseconds).  The
    timed launches run back to back (no cache flush) between two HIP events
    on the stream the kernels run on; ``ms_per_step`` is their mean.  A
    second pass of as many launches, with an event between consecutive
    launches, gives the per-launch latencies (an event between launches adds
    a few microseconds to each, which matters only for short kernels)."""
    import numpy as np
    import torch
    import exact_attention_112_amd as fa
    from exact_attention_112_amd import inputs as I

    print(f"bench: generating inputs for {w.name}", file=sys.stderr, flush=True)
    inp = I.make_inputs(w)
    if w.dtype == "bf16":
        up = lambda bits: torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to("cuda")
        tq, tk, tv = up(inp.q_bits), up(inp.k_bits), up(inp.v_bits)
    else:
        tq, tk, tv = (torch.from_numpy(x).to("cuda") for x in (inp.q, inp.k, inp.v))
    out_dtype = torch.bfloat16 if args.out_dtype == "bf16" else torch.float32
    o = torch.empty(tq.shape, dtype=out_dtype, device="cuda")
    lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device="cuda")

    bmask, sparse_flops = None, None
    if w.block_sparse:
        mask_np = I.make_block_mask(w)
        bmask = torch.from_numpy(mask_np).to("cuda")
        sparse_flops = sparse_pair_flops(w, mask_np)

    def step():
        fa.fwd(tq, tk, tv, causal=w.causal, scale=w.scale, layout=w.layout, out_dtype=out_dtype,
               out=o, lse=lse, window=None if w.window == (-1, -1) else w.window, block_mask=bmask)

    if args.which == "bwd":
        if w.dtype != "bf16":
            print("bench.py: the backward pass takes bf16 inputs", file=sys.stderr)
            return None
        grad_vals, grad_bits = I.make_grad(w)
        tdo = up(grad_bits)
        step()                                   # O and LSE for the backward, untimed
        dq = torch.empty(tq.shape, dtype=torch.float32, device="cuda")
        dk = torch.empty(tk.shape, dtype=torch.float32, device="cuda")
        dv = torch.empty(tk.shape, dtype=torch.float32, device="cuda")
        delta = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device="cuda")

        def step():  # noqa: F811  (the timed step of the backward benchmark)
            fa.bwd(tq, tk, tv, o, tdo, lse, causal=w.causal, scale=w.scale, layout=w.layout,
                   window=None if w.window == (-1, -1) else w.window, block_mask=bmask, dq=dq, dk=dk, dv=dv,
                   delta=delta)

    print(f"bench: warmup {warmup}", file=sys.stderr, flush=True)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    if min_warmup_s > 0:
        t_w = time.perf_counter()
        while time.perf_counter() - t_w < min_warmup_s:
            for _ in range(20):
                step()
            torch.cuda.synchronize()
    stream = torch.cuda.current_stream()        # the stream fa.fwd / fa.bwd launch on
    print(f"bench: timing {steps} steps", file=sys.stderr, flush=True)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    # per-launch latencies: a second pass with an event between launches
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(stream)
    for i in range(steps):
        step()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    srt = sorted(per)
    latency = {"mean": round(sum(per) / steps, 4), "median": round(srt[len(srt) // 2] if len(srt) % 2 else
                                                     0.5 * (srt[len(srt) // 2 - 1] + srt[len(srt) // 2]), 4),
               "min": round(srt[0], 4), "max": round(srt[-1], 4)}
    bwd = args.which == "bwd"
    fwd_flops = sparse_flops if w.block_sparse else w.flops
    flops = 2.5 * fwd_flops if bwd else fwd_flops
    tflops = flops / (ms * 1e-3) / 1e12
    outs = (dq, dk, dv) if bwd else (o, lse)
    if not all(torch.isfinite(t).all() for t in outs):
        print("bench: non-finite output", file=sys.stderr)
        return None

    cpu = None
    if with_cpu:
        print("bench: timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        if bwd and w.block_sparse:
            cpu = cpu_baseline_bwd_sparse(w, inp, grad_vals, mask_np)
        elif bwd:
            cpu = cpu_baseline_bwd(w, inp, grad_vals)
        elif w.block_sparse:
            cpu = cpu_baseline_sparse(w, inp, mask_np)
        else:
            cpu = cpu_baseline(w, inp)

    traffic = traffic_from_profiles(w.name, args.which)
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    nbytes = bwd_algorithmic_bytes(w) if bwd else algorithmic_bytes(w, 2 if args.out_dtype == "bf16" else 4)
    if flops / nbytes < peak * 1e12 / (PEAK_HBM_GBS * 1e9):
        gbs = nbytes / (ms * 1e-3) / 1e9     # below the ridge point: HBM-bound
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": traffic}
    else:
        roof = {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(tflops / peak, 4), "traffic": traffic}
    line = {
        "metric": ((BWD_METRIC if bwd else METRIC) if w.name == "selfattn_b4h32n8k"
                   else f"attention {args.which} TFLOPS and % of bf16 MFMA peak at {w.name}"),
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": ("synthetic (seeded N(0,1) Q/K/V/dO of the workload's shape, seeded BigBird-like block mask; "
                 "O, LSE from the GPU forward)" if w.block_sparse and bwd else
                 "synthetic (seeded N(0,1) Q/K/V of the workload's shape, seeded BigBird-like block mask)"
                 if w.block_sparse else
                 "synthetic (seeded N(0,1) Q/K/V/dO of the workload's shape; O, LSE from the GPU forward)"
                 if bwd else "synthetic (seeded N(0,1) Q/K/V of the workload's shape)"),
        "config": {"workload": w.name, "B": w.B, "H": w.H, "Nq": w.Nq, "Nk": w.Nk, "d": w.d,
                   "causal": w.causal, "layout": w.layout, "out_dtype": args.out_dtype,
                   **({"Hkv": w.kv_heads, "window": list(w.window)}
                      if w.kv_heads != w.H or w.window != (-1, -1) else {}),
                   **({"block_sparse": True, "mask_density": round(float(mask_np.mean()), 4)}
                      if w.block_sparse else {}),
                   **({"pass": "bwd", "grads": "f32"} if bwd else {})},
        "latency_ms": latency,
        "tflops_at_median": round(flops / (latency["median"] * 1e-3) / 1e12, 2),
        "roofline": roof,
        "counters": counters_from_profiles(w.name, args.which),
        "cpu_baseline": cpu,
        "context": {"peak_note": "MI355X published dense peaks: bf16 MFMA 2.5 PFLOP/s, HBM 8 TB/s",
                    "pages": PAGES_CONTEXT},
    }
    return line


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="selfattn_b4h32n8k",
                    help="a workload name, or 'all' for the five forward workloads one after another")
    ap.add_argument("--out-dtype", default="f32", choices=["f32", "bf16"])
    ap.add_argument("--pass", dest="which", default="fwd", choices=["fwd", "bwd"],
                    help="time the forward pass (default) or the backward pass")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle timing (for profiler runs)")
    ap.add_argument("--min-warmup-s", type=float, default=0.0, metavar="SECONDS",
                    help="keep warming up past --warmup calls until this much time has passed (short "
                         "kernels: the clock ramps up over tens of milliseconds); --workload all uses 1")
    ap.add_argument("--out", default=None, metavar="PATH",
                    help="with --workload all: also write every record to this JSON file")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES bytes 3 times (the "
                         "reference for scaling HBM counters), then exit")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py: the benchmark runs on one GPU; --gpus {args.gpus} is not supported "
              "(heads are independent: the path would shard by heads across GPUs)", file=sys.stderr)
        return 2

    import numpy as np
    import torch
    import exact_attention_112_amd as fa
    from exact_attention_112_amd import inputs as I

    if not torch.cuda.is_available():
        print("bench.py: no GPU", file=sys.stderr)
        return 1
    if args.calibrate_copy:
        n = args.calibrate_copy // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n * 4}), flush=True)
        return 0
    fa.load()
    if args.workload in I.DECODE_WORKLOADS:
        return bench_decode(args, I.DECODE_WORKLOADS[args.workload])
    names = FORWARD_WORKLOADS if args.workload == "all" else [args.workload]
    if args.workload == "all" and args.which != "fwd":
        print("bench.py: --workload all times the forward pass", file=sys.stderr)
        return 2
    if args.workload == "all":
        records = []
        for name in names:
            w = I.WORKLOADS[name]
            steps, warmup = (10, 2) if w.Nq >= 65536 else (30, 5)
            rec = bench_attention(args, w, steps, warmup, with_cpu=not args.no_cpu_baseline,
                                  min_warmup_s=max(1.0, args.min_warmup_s))
            if rec is None:
                return 1
            print(json.dumps(rec), flush=True)
            records.append(rec)
        if args.out:
            with open(args.out, "w") as f:
                json.dump({"records": records}, f, indent=1)
        return 0
    rec = bench_attention(args, I.WORKLOADS[args.workload], args.steps, args.warmup,
                          with_cpu=not args.no_cpu_baseline, min_warmup_s=args.min_warmup_s)
    if rec is None:
        return 1
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

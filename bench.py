#!/usr/bin/env python3
"""Throughput of weight-absorbed MLA paged decode on one MI355X.

One step = one decode call over one batch: the main kernel (mla_decode_fwd)
and the merge of split row blocks (mla_combine), with the split plan built on
the host once per batch (a serving step reuses it for every layer; its host
time is reported separately).  Inputs are seeded synthetic tensors with the
workload's shapes, already resident in HBM.  Consecutive steps rotate over
several copies of the inputs whose total size is well above the 256 MB
Infinity Cache, so every step streams its cache from HBM.

Prints ONE JSON line:
  value       KV GB/s: cached latent bytes of the visible keys / device time per step
  us_per_call device time per step (fwd + combine), from HIP events (mean;
              us_per_call_pct and us_fwd_kernel_pct give p10 / median / p90)
  roofline    dominant kernel (mla_decode_kernel): algorithmic bytes (or FLOPs)
              per launch / its average launch time, against MI355X peak
  cpu_baseline the float64 oracle on a bounded sample of the same workload

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

The append_* workloads instead time the cache append (mla_kv_append) alone:
one decode step's new tokens, or a prompt's worth per sequence.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MLA decode µs/call, KV HBM GB/s and % of roofline at DeepSeek-V3 shapes"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 MFMA
MALL_BYTES = 256 << 20
KERNEL_SOURCES = ("decode_kernel.hip", "gfx950_asm.h", "kernels.h", "plan_layout.h")
DECODE_KERNEL = "mla_decode_kernel"
# the kernel a plan launches: a bf16 cache with one workgroup per 128-row block
# runs the 32-key kernel, every other plan the 16-key one
PAIRS_KERNEL = "mla_decode_kernel_pairs"


W8_KERNEL = "mla_decode_kernel_w8"
QRES_KERNEL = "mla_decode_kernel_qres"
SPLIT_KERNEL = "mla_decode_kernel_split"


def _w8_selected(kv_dtype: str, phases: int) -> bool:
    return os.environ.get("MLA_DECODE_KERNEL") == "w8" and phases == 1


def _qres_selected(kv_dtype: str) -> bool:
    return os.environ.get("MLA_DECODE_KERNEL") == "qres" and kv_dtype != "bf16"


def _split_selected(kv_dtype: str, phases: int) -> bool:
    return os.environ.get("MLA_DECODE_KERNEL") == "split" and phases == 1


def decode_kernel_name(kv_dtype: str, phases: int) -> str:
    if _w8_selected(kv_dtype, phases):
        return W8_KERNEL
    if _qres_selected(kv_dtype):
        return QRES_KERNEL
    if _split_selected(kv_dtype, phases):
        return SPLIT_KERNEL
    return PAIRS_KERNEL if kv_dtype == "bf16" and phases == 1 else DECODE_KERNEL


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


APPEND_SOURCES = ("append_kernel.hip", "append.h", "plan_layout.h")


def kernel_source_hash(sources=KERNEL_SOURCES) -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "mla_paged_decode_absorbed_amd", "csrc")
    for name in sources:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _blas_threads() -> int:
    """Threads of numpy's BLAS (the oracle's matrix products), 1 if unknown."""
    try:
        import threadpoolctl
    except ImportError:  # pragma: no cover
        return 1
    info = [i for i in threadpoolctl.threadpool_info() if i.get("user_api") == "blas"]
    return int(info[0].get("num_threads", 1)) if info else 1


def workload_counts(case):
    """Algorithmic bytes and FLOPs of one decode call.

    Bytes: every visible cached row once (bf16: 1152 B; e4m3: 576 B + a 4 B
    scale), every valid query row (1152 B), output row (1024 B) and LSE (4 B),
    the block-table entries in use and the two length arrays.
    FLOPs: 2 * (576 + 512) per (query row, visible key)."""
    H, D, Dv, P = case.num_heads, case.d_qk, case.d_latent, case.page_size
    kv_row = D * 2 if case.kv_dtype == "bf16" else D + 4
    kv_tokens = int(case.kv_lens.astype("int64").sum())
    rows = int(case.q_lens.astype("int64").sum()) * H
    pages = sum((int(L) + P - 1) // P for L in case.kv_lens)
    kv_bytes = kv_tokens * kv_row
    other = rows * (D * 2 + Dv * 2 + 4) + pages * 4 + case.batch * 8
    visible = 0
    for L, qb in zip(case.kv_lens, case.q_lens):
        for t in range(int(qb)):
            visible += max(0, int(L) - int(qb) + t + 1) if case.causal else int(L)
    flops = 2 * visible * H * (D + Dv)
    return dict(kv_bytes=kv_bytes, alg_bytes=kv_bytes + other, flops=flops,
                kv_tokens=kv_tokens, rows=rows)


def code_object_hash(source: str, kernel: str):
    """Fingerprint of one kernel in the built library (its machine code,
    kernel descriptor and metadata, as the build records them), or None."""
    path = os.path.join(ROOT, "mla_paged_decode_absorbed_amd", "_build", "code_objects.json")
    try:
        with open(path) as f:
            return (json.load(f).get(source) or {}).get(kernel)
    except (OSError, ValueError, AttributeError):
        return None


def decode_kernel_symbol(kv_dtype: str, phases: int) -> str:
    """The instantiation a plan launches, as the build's fingerprints name it."""
    if _w8_selected(kv_dtype, phases):
        return f"mla_decode_kernel_w8<{0 if kv_dtype == 'bf16' else 1}>"
    if _qres_selected(kv_dtype):
        return f"mla_decode_kernel_qres<1, {phases}>"
    if _split_selected(kv_dtype, phases):
        return f"mla_decode_kernel_split<{0 if kv_dtype == 'bf16' else 1}>"
    if kv_dtype == "bf16" and phases == 1:
        return "mla_decode_kernel_pairs<0>"
    return f"mla_decode_kernel<{0 if kv_dtype == 'bf16' else 1}, {phases}>"


def percentiles(ms):
    """p10 / median / p90 of per-launch times in ms, returned in microseconds."""
    xs = sorted(ms)
    n = len(xs)

    def q(p):   # linear interpolation between order statistics
        x = p * (n - 1)
        i = int(math.floor(x))
        j = min(i + 1, n - 1)
        return xs[i] + (xs[j] - xs[i]) * (x - i)

    return {"p10": round(q(0.1) * 1e3, 2), "median": round(q(0.5) * 1e3, 2),
            "p90": round(q(0.9) * 1e3, 2)}


def read_traffic(workload: str, kernel: str = DECODE_KERNEL, sources=KERNEL_SOURCES,
                 symbol: str | None = None):
    """HBM bytes per launch of a kernel from the committed counter summary, or
    None if there is none or the kernel changed since.  A summary keyed by
    code_object_sha256 holds while the fingerprint of `symbol` (the launched
    instantiation, in sources[0]) is the one it was counted on; an older one
    keyed by kernel_source_sha256 holds while the source text is unchanged."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if "code_object_sha256" in kv:
        if symbol is None or kv["code_object_sha256"] != code_object_hash(sources[0], symbol):
            return None
    elif kv.get("kernel_source_sha256") != kernel_source_hash(sources):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(case, seconds: float, kv_bytes_total: int, seq_fn=None):
    """Time the float64 oracle on the sequences of the same workload, taken in
    order (and cycling) until ``seconds`` have passed.  ``seq_fn(b)`` replaces
    the decode oracle of one sequence (the tree-draft oracle, for instance)."""
    import numpy as np

    import oracle

    done = 0
    tokens = 0
    order = [b for b in range(case.batch) if int(case.q_lens[b]) > 0]
    t0 = time.perf_counter()
    while order and time.perf_counter() - t0 < seconds:
        b = order[done % len(order)]
        if seq_fn is None:
            oracle.mla_decode_ref_seq(case, b)
        else:
            seq_fn(b)
        done += 1
        tokens += int(case.kv_lens[b])
    el = time.perf_counter() - t0
    threads = _blas_threads()
    row = case.d_qk * 2 if case.kv_dtype == "bf16" else case.d_qk + 4
    gbs = tokens * row / el / 1e9
    frac = tokens * row / kv_bytes_total
    return {
        "value": round(gbs, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
        "sample": (f"float64 numpy oracle, {done} sequence evaluations taken in order "
                   f"(cycling) from the {case.batch} of the workload = {frac:.2f}x its KV "
                   f"tokens, in {el:.1f} s; "
                   f"os.cpu_count()={os.cpu_count()}, affinity={len(os.sched_getaffinity(0))}"),
        "us_per_call_equiv": round(el / max(frac, 1e-12) * 1e6, 1),
    }


APPEND_KERNEL = "mla_kv_append_kernel"
APPEND_WORKLOADS = {
    # name: (sequences, new tokens per sequence, cached tokens per sequence, kv dtype)
    "append_step_v3_bf16": (64, 1, 2560, "bf16"),
    "append_prompt_bf16": (64, 2560, 2560, "bf16"),
    "append_prompt_fp8": (64, 2560, 2560, "fp8_e4m3"),
}


def append_counts(B, n, kv_dtype, page_size=64):
    """Algorithmic bytes of one append: each new row read once (1152 B) and
    written once (bf16 1152 B; e4m3 576 B + a 4 B scale), one block-table
    entry per page touched, the two length arrays."""
    rows = B * n
    written = 1152 if kv_dtype == "bf16" else 576 + 4
    pages = B * ((n + page_size - 1) // page_size)
    return dict(rows=rows, alg_bytes=rows * (1152 + written) + pages * 4 + B * 8)


def append_cpu_baseline(rows_np, kv_dtype, seconds: float):
    """The oracle's append on a bounded sample: chunks of (up to) 256 rows of
    the workload, taken in order, each appended as one sequence's new tokens
    into a cache of that many slots, until ``seconds`` pass."""
    import numpy as np

    from oracle import append_ref

    n = rows_np.shape[0]
    P, chunk = 64, min(256, n)
    pages = (chunk + P - 1) // P
    kv = np.zeros((pages, P, 576), np.uint16 if kv_dtype == "bf16" else np.uint8)
    sc = None if kv_dtype == "bf16" else np.zeros((pages, P), np.float32)
    bt = np.arange(pages, dtype=np.int32)[None, :]
    lens = np.array([chunk], np.int32)
    done = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        k0 = (done * chunk) % max(1, n - chunk + 1)
        block = rows_np[None, k0:k0 + chunk]
        kv, sc, _ = append_ref.kv_append_ref(kv, sc, bt, lens, lens, block, P, kv_dtype)
        done += 1
    el = time.perf_counter() - t0
    rows_done = done * chunk
    written = 1152 if kv_dtype == "bf16" else 580
    return {
        "value": round(rows_done * (1152 + written) / el / 1e9, 4), "unit": "GB/s", "cores": 1,
        "kind": "oracle",
        "sample": (f"numpy oracle append, {rows_done} rows of the workload in chunks of "
                   f"{chunk}, each into a {pages}-page cache, in {el:.1f} s"),
    }


def main_append(args) -> int:
    import numpy as np
    import torch

    import mla_paged_decode_absorbed_amd as mla

    B, n, L, kv_dtype = APPEND_WORKLOADS[args.workload]
    P = 64
    dev = torch.device("cuda:0")
    mla.load_library()
    cnt = append_counts(B, n, kv_dtype, P)
    log(f"workload {args.workload}: {B} sequences x {n} new tokens ({cnt['rows']} rows)")
    rng = np.random.default_rng(2)
    pages_per_seq = (L + P - 1) // P
    pool = B * pages_per_seq
    bt_np = rng.permutation(pool).astype(np.int32).reshape(B, pages_per_seq)
    kv_lens_np = np.full(B, L, np.int32)
    new_np = np.full(B, n, np.int32)
    rows32 = (rng.standard_normal((B * n, 576), dtype=np.float32) * 0.5)
    rows_bits = torch.from_numpy(rows32).to(torch.bfloat16).view(torch.int16).numpy()
    kvd = mla.KV_BF16 if kv_dtype == "bf16" else mla.KV_FP8_E4M3
    shape = mla.Shape.make(batch=B, num_heads=128, max_q_len=1, page_size=P, num_pages=pool,
                           max_pages_per_seq=pages_per_seq, kv_dtype=kvd)
    row_bytes = 1152 if kv_dtype == "bf16" else 576
    set_bytes = B * n * 1152 + pool * P * row_bytes
    nsets = max(2, math.ceil(3 * MALL_BYTES / set_bytes))
    sets = []
    for _ in range(nsets):
        src = torch.from_numpy(rows_bits).view(torch.bfloat16).to(dev).view(B, n, 576)
        if kv_dtype == "bf16":
            kv = torch.empty((pool, P, 576), dtype=torch.int16, device=dev)
            sc = None
        else:
            kv = torch.empty((pool, P, 576), dtype=torch.uint8, device=dev)
            sc = torch.empty((pool, P), dtype=torch.float32, device=dev)
        sets.append((src, kv, sc))
    bt = torch.from_numpy(bt_np).to(dev)
    kvl = torch.from_numpy(kv_lens_np).to(dev)
    nl = torch.from_numpy(new_np).to(dev)
    stream = torch.cuda.current_stream()

    def step(k):
        src, kv, sc = sets[k % nsets]
        mla.kv_append(shape, src, bt, kvl, kv, new_lens=nl, kv_scale=sc, stream=stream)

    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
    w0 = time.perf_counter()
    for k in range(K):
        ev[k][0].record(stream)
        step(k)
        ev[k][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    call_ms = [ev[k][0].elapsed_time(ev[k][1]) for k in range(K)]
    avg_ms = sum(call_ms) / K
    t = avg_ms * 1e-3
    achieved = cnt["alg_bytes"] / t / 1e9
    log(f"timed {K} appends: avg {avg_ms * 1e3:.2f} us, {achieved:.1f} GB/s")
    append_sym = f"{APPEND_KERNEL}<{0 if kv_dtype == 'bf16' else 1}>"
    traffic = read_traffic(args.workload, APPEND_KERNEL, APPEND_SOURCES, append_sym)
    res = {
        "metric": "MLA cache append µs/call and HBM GB/s",
        "value": round(achieved, 2), "unit": "GB/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(avg_ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if kv_dtype == "bf16" else "bf16->e4m3", "data": "synthetic",
        "config": {"workload": args.workload, "batch": B, "new_tokens_per_seq": n,
                   "kv_len": L, "page_size": P, "kv_dtype": kv_dtype},
        "us_per_call": round(avg_ms * 1e3, 2),
        "us_per_call_pct": percentiles(call_ms),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None if traffic is None else round(traffic),
                     "kernel": APPEND_KERNEL, "alg_bytes_per_launch": cnt["alg_bytes"]},
        "wall_s_timed": round(wall, 4), "input_sets": nsets,
        "kernel_source_sha256": kernel_source_hash(APPEND_SOURCES),
        "code_object_sha256": code_object_hash(APPEND_SOURCES[0], append_sym),
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log(f"cpu baseline: oracle append for about {args.cpu_seconds:.0f} s")
        res["cpu_baseline"] = append_cpu_baseline(rows_bits.view(np.uint16), kv_dtype,
                                                  args.cpu_seconds)
    print(json.dumps(res), flush=True)
    return 0


PREFILL_KERNEL = "mla_prefill_attn_kernel"
PREFILL_SOURCES = ("prefill_attn_kernel.hip", "prefill.h")
MFMA_INT8_FP8_PEAK_TOPS = 5000.0   # dense INT8 and FP8 MFMA, MI355X


def prefill_counts(seqlens, H):
    """Work of one quantized causal prefill.

    Ops: every (query, visible key) pair of a head costs 2 * 192 (INT8 QK) +
    2 * 128 (e4m3 PV).  Quantize bytes: bf16 Q, K, V read once; INT8 codes of
    Q and K with Q's per-row and K's per-block fp32 scales, e4m3 V codes and
    per-block channel scales written.  Attention bytes: codes and scales read
    once, bf16 O and fp32 LSE written."""
    lens = [int(n) for n in seqlens]
    pairs = sum(n * (n + 1) // 2 for n in lens)
    T = sum(lens)
    nb = sum((n + 127) // 128 for n in lens)
    return {
        "tokens": T, "blocks": nb, "pairs": pairs * H,
        "ops": pairs * H * 2 * (192 + 128),
        "quant_bytes": T * H * (2 * 192 * 2 + 128 * 2) + T * H * (2 * 192 + 4) + nb * H * 4
        + nb * H * 128 * (128 + 4),
        "attn_bytes": T * H * (2 * 192 + 4) + nb * H * 4 + nb * H * 128 * (128 + 4)
        + T * H * (256 + 4),
    }


def prefill_cpu_baseline(case, seconds: float, ops_total: int):
    """The float64 oracle on one head of the same prompt: its quantizers, then
    sampled rows (random tokens), until ``seconds`` have passed; scaled to
    the whole workload's tokens/s by the share of its ops done."""
    import numpy as np
    from oracle import prefill_ref
    from workloads.prefill import PrefillCase
    t0 = time.perf_counter()
    one = PrefillCase(name="one-head", seqlens=case.seqlens, cu_seqlens=case.cu_seqlens,
                      num_heads=1, sm_scale=case.sm_scale, q=case.q[:, :1], k=case.k[:, :1],
                      v=case.v[:, :1])
    quant = prefill_ref.quantize_case(one)
    rng = np.random.default_rng(0)
    cu = case.cu_seqlens
    ops = 0
    rows = 0
    while time.perf_counter() - t0 < seconds:
        t = int(rng.integers(0, case.num_tokens))
        prefill_ref.sage_prefill_ref(one, rows=[(t, 0)], quantized=quant)
        s = int(np.searchsorted(cu, t, side="right") - 1)
        ops += (t - int(cu[s]) + 1) * 2 * (192 + 128)
        rows += 1
    el = time.perf_counter() - t0
    return {"value": round(case.num_tokens * (ops / ops_total) / el, 6), "unit": "tokens/s",
            "cores": _blas_threads(), "kind": "oracle",
            "sample": f"one head of the same prompt quantized, then {rows} random query rows "
                      f"({ops:.3g} of the workload's {ops_total:.3g} ops) in {el:.1f} s, "
                      f"scaled by the share of ops done"}


def main_prefill(args) -> int:
    import numpy as np
    import torch

    import mla_paged_decode_absorbed_amd as mla
    from workloads.prefill import PREFILL_WORKLOADS, prefill_workload

    dev = torch.device("cuda:0")
    mla.load_library()
    log(f"workload {args.workload}: generating inputs")
    case = prefill_workload(args.workload)
    H = case.num_heads
    cnt = prefill_counts(case.seqlens, H)
    shape = mla.PrefillShape.make(case.seqlens, H)

    def bf16(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v = bf16(case.q), bf16(case.k), bf16(case.v)
    cu = torch.from_numpy(case.cu_seqlens.astype(np.int32)).to(dev)
    quant = mla.prefill_alloc_quant(shape, dev)
    out = torch.empty((case.num_tokens, H, 128), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((case.num_tokens, H), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    log(f"{case.num_seqs} prompts, {cnt['tokens']} tokens, {H} heads, {cnt['blocks']} blocks")

    def step():
        mla.prefill_quantize(shape, cu, q, k, v, quant=quant, stream=stream)

    def step_attn():
        mla.prefill_attn(shape, cu, quant, case.sm_scale, out=out, lse=lse, stream=stream)

    for _ in range(args.warmup):
        step()
        step_attn()
    torch.cuda.synchronize()
    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    w0 = time.perf_counter()
    for i in range(K):
        ev[i][0].record(stream)
        step()
        ev[i][1].record(stream)
        step_attn()
        ev[i][2].record(stream)
        if (i + 1) % 10 == 0:
            torch.cuda.synchronize()
            log(f"step {i + 1}/{K}")
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    a_list = [e[1].elapsed_time(e[2]) for e in ev]
    q_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / K
    a_ms = sum(a_list) / K
    call_ms = q_ms + a_ms
    tops = cnt["ops"] / (a_ms * 1e-3) / 1e12
    quant_gbs = cnt["quant_bytes"] / (q_ms * 1e-3) / 1e9
    log(f"timed {K} calls: quantize {q_ms:.3f} ms ({quant_gbs:.0f} GB/s), "
        f"attention {a_ms:.3f} ms ({tops:.1f} TOPS)")
    prefill_sym = f"{PREFILL_KERNEL}<4, 1>"
    traffic = read_traffic(args.workload, PREFILL_KERNEL, PREFILL_SOURCES, prefill_sym)
    res = {
        "metric": "quantized causal prefill tokens/s (INT8 QK, e4m3 PV, head dim 192/128)",
        "value": round(cnt["tokens"] / (call_ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": K, "warmup": args.warmup, "ms_per_step": round(call_ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "int8+e4m3", "data": "synthetic",
        "config": {"workload": args.workload, "prompts": case.num_seqs, "tokens": cnt["tokens"],
                   "num_heads": H, "d_qk": 192, "d_v": 128, "causal": True,
                   "description": PREFILL_WORKLOADS[args.workload][1]},
        "ms_quantize": round(q_ms, 4), "ms_attention": round(a_ms, 4),
        "us_attention_pct": percentiles(a_list),
        "quantize_GBps": round(quant_gbs, 1), "attention_tops": round(tops, 2),
        "roofline": {"bound": "mfma", "achieved": round(tops, 2),
                     "peak": MFMA_INT8_FP8_PEAK_TOPS, "unit": "TOPS",
                     "frac": round(tops / MFMA_INT8_FP8_PEAK_TOPS, 4),
                     "traffic": None if traffic is None else round(traffic),
                     "kernel": PREFILL_KERNEL, "ops_per_launch": cnt["ops"],
                     "alg_bytes_per_launch": cnt["attn_bytes"]},
        "wall_s_timed": round(wall, 4),
        "kernel_source_sha256": kernel_source_hash(PREFILL_SOURCES),
        "code_object_sha256": code_object_hash(PREFILL_SOURCES[0], prefill_sym),
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log(f"cpu baseline: oracle on one head for about {args.cpu_seconds:.0f} s")
        res["cpu_baseline"] = prefill_cpu_baseline(case, args.cpu_seconds, cnt["ops"])
    print(json.dumps(res), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="v3_decode_bf16")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="also time mla_decode_fwd + mla_combine replayed from HIP graphs "
                         "captured with a fixed-shape plan (us_per_call_graph)")
    ap.add_argument("--num-workgroups", type=int, default=0,
                    help="plan the decode for this many workgroups instead of one per CU "
                         "(per-CU throughput against the number of CUs at work)")
    ap.add_argument("--decode-kernel", choices=("default", "w8", "qres", "split"),
                    default="default",
                    help="w8: time the two-waves-per-SIMD candidate with 16 rows per wave "
                         "(one-phase plans, bf16 or e4m3 cache); split: the one whose pairs of "
                         "waves share 32 rows (likewise); qres: the library's e4m3 kernels with Q "
                         "resident before the key loop (e4m3 caches); none has run on a GPU yet")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB --steps times "
                         "(scales HBM byte counters against a kernel of known traffic)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this decode path runs on a single MI355X "
              "(sharding by sequence is a design note, not built). Use --gpus 1.",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import mla_paged_decode_absorbed_amd as mla
    from workloads import workload

    if args.decode_kernel != "default":
        os.environ["MLA_DECODE_KERNEL"] = args.decode_kernel
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.workload in APPEND_WORKLOADS:
        return main_append(args)
    from workloads.prefill import PREFILL_WORKLOADS
    if args.workload in PREFILL_WORKLOADS:
        return main_prefill(args)
    if args.copy_calib_mib > 0:
        n = args.copy_calib_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(max(1, args.steps)):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration": True, "bytes_read_per_copy": n,
                          "bytes_written_per_copy": n, "copies": max(1, args.steps)}))
        return 0
    mla.load_library()

    log(f"workload {args.workload}: generating inputs")
    case = workload(args.workload)
    full = case
    tree = case.meta.get("tree_mask")
    if tree is not None:
        # tree-shaped drafts: the decode kernels run over the cached prefix
        # (kv_len - q_len keys, non-causal) and mla_tree_attend adds the drafts
        import dataclasses
        case = dataclasses.replace(full, kv_lens=(full.kv_lens - full.q_lens).astype(np.int32),
                                   causal=False)
    cnt = workload_counts(case)
    kv_total = workload_counts(full)["kv_bytes"]
    kvd = mla.KV_BF16 if case.kv_dtype == "bf16" else mla.KV_FP8_E4M3
    shape = mla.Shape.make(batch=case.batch, num_heads=case.num_heads, max_q_len=case.max_q_len,
                           page_size=case.page_size, num_pages=case.num_pages,
                           max_pages_per_seq=case.max_pages, kv_dtype=kvd, causal=case.causal)
    nwg = args.num_workgroups if args.num_workgroups > 0 else None
    t0 = time.perf_counter()
    for _ in range(20):
        pl = mla.plan(shape, case.kv_lens, case.q_lens, num_workgroups=nwg, device=dev,
                      upload=False)
    plan_us = (time.perf_counter() - t0) / 20 * 1e6
    pl = mla.plan(shape, case.kv_lens, case.q_lens, num_workgroups=nwg, device=dev)

    # input sets: enough copies that consecutive steps miss the Infinity Cache
    kv_np = case.kv.view(np.int16) if case.kv_dtype == "bf16" else case.kv
    set_bytes = case.kv.nbytes + case.q.nbytes + case.batch * case.max_q_len * case.num_heads * 1024
    nsets = max(2, math.ceil(3 * MALL_BYTES / set_bytes))
    sets = []
    for _ in range(nsets):
        q = torch.from_numpy(case.q.view(np.int16)).view(torch.bfloat16).to(dev)
        kv = torch.from_numpy(kv_np).to(dev)
        if case.kv_dtype == "bf16":
            kv = kv.view(torch.bfloat16)
        sc = None if case.kv_scale is None else torch.from_numpy(case.kv_scale).to(dev)
        bt = torch.from_numpy(case.block_table).to(dev)
        kvl = torch.from_numpy(case.kv_lens).to(dev)
        ql = torch.from_numpy(case.q_lens).to(dev)
        out = torch.empty((case.batch, case.max_q_len, case.num_heads, 512), dtype=torch.bfloat16,
                          device=dev)
        lse = torch.empty((case.batch, case.max_q_len, case.num_heads), dtype=torch.float32,
                          device=dev)
        sets.append((q, kv, sc, bt, kvl, ql, out, lse))
    if tree is not None:
        kvl_full = torch.from_numpy(full.kv_lens).to(dev)
        mask_d = torch.from_numpy(np.asarray(tree, np.uint32).view(np.int32)).to(dev)
    ws = mla.alloc_workspace(pl, dev) if pl.info.num_partials > 0 else None
    stream = torch.cuda.current_stream()
    log(f"plan: {pl.info.num_workgroups} workgroups, {pl.info.num_items} items, "
        f"{pl.info.num_partials} partials, {pl.info.num_combine} combine; {nsets} input sets")

    def step(k):
        q, kv, sc, bt, kvl, ql, out, lse = sets[k % nsets]
        mla.decode_fwd(shape, pl, q, kv, bt, kvl, ql, case.sm_scale, out, lse, ws, kv_scale=sc,
                       stream=stream)

    def step_combine(k):
        q, kv, sc, bt, kvl, ql, out, lse = sets[k % nsets]
        mla.combine(shape, pl, ws, ql, out, lse, stream=stream)
        if tree is not None:
            mla.tree_attend(shape, q, kv, bt, kvl_full, ql, mask_d, case.sm_scale, out, lse,
                            kv_scale=sc, stream=stream)

    for k in range(args.warmup):
        step(k)
        step_combine(k)
    torch.cuda.synchronize()

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    for k in range(K):
        ev[k][0].record(stream)
        step(k)
        ev[k][1].record(stream)
        step_combine(k)
        ev[k][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    fwd_ms = [ev[k][0].elapsed_time(ev[k][1]) for k in range(K)]
    step_ms = [ev[k][0].elapsed_time(ev[k][2]) for k in range(K)]
    fwd_avg = sum(fwd_ms) / K
    step_avg = sum(step_ms) / K
    log(f"timed {K} steps: wall {wall * 1e3:.2f} ms, fwd avg {fwd_avg * 1e3:.2f} us, "
        f"step avg {step_avg * 1e3:.2f} us")

    # warm reference: one input set, the Infinity Cache may hold the cache
    warm = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
    for k in range(K):
        warm[k][0].record(stream)
        step(0)
        step_combine(0)
        warm[k][1].record(stream)
    torch.cuda.synchronize()
    warm_avg = sum(warm[k][0].elapsed_time(warm[k][1]) for k in range(K)) / K

    tree_avg = None
    if tree is not None:
        tev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
        for k in range(K):
            q, kv, sc, bt, kvl, ql, out, lse = sets[k % nsets]
            tev[k][0].record(stream)
            mla.tree_attend(shape, q, kv, bt, kvl_full, ql, mask_d, case.sm_scale, out, lse,
                            kv_scale=sc, stream=stream)
            tev[k][1].record(stream)
        torch.cuda.synchronize()
        tree_avg = sum(tev[k][0].elapsed_time(tev[k][1]) for k in range(K)) / K
        log(f"tree merge: avg {tree_avg * 1e3:.2f} us")

    graph_avg = plan_dev_us = None
    if args.graph and tree is None:
        # one graph per input set, each capturing fwd + combine with the
        # fixed-shape plan of the same lengths (same split, all workgroups)
        plf = mla.plan(shape, case.kv_lens, case.q_lens, num_workgroups=nwg, device=dev,
                       fixed=True)
        wsf = torch.empty(plf.info.workspace_bytes, dtype=torch.uint8, device=dev)
        graphs = []
        for k in range(nsets):
            q, kv, sc, bt, kvl, ql, out, lse = sets[k]
            mla.decode_fwd(shape, plf, q, kv, bt, kvl, ql, case.sm_scale, out, lse, wsf,
                           kv_scale=sc)
            mla.combine(shape, plf, wsf, ql, out, lse)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                mla.decode_fwd(shape, plf, q, kv, bt, kvl, ql, case.sm_scale, out, lse, wsf,
                               kv_scale=sc)
                mla.combine(shape, plf, wsf, ql, out, lse)
            graphs.append(g)
        torch.cuda.synchronize()
        for k in range(args.warmup):
            graphs[k % nsets].replay()
        torch.cuda.synchronize()
        gev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
        for k in range(K):
            gev[k][0].record(stream)
            graphs[k % nsets].replay()
            gev[k][1].record(stream)
        torch.cuda.synchronize()
        graph_avg = sum(gev[k][0].elapsed_time(gev[k][1]) for k in range(K)) / K
        log(f"graph replays: avg {graph_avg * 1e3:.2f} us per fwd + combine")
        # the device-side planner on the same lengths (one workgroup)
        kvl0, ql0 = sets[0][4], sets[0][5]
        dp = mla.plan_device(shape, kvl0, ql0, num_workgroups=nwg)
        for _ in range(3):
            mla.plan_device(shape, kvl0, ql0, plan_buf=dp.device, num_workgroups=nwg)
        torch.cuda.synchronize()
        pev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(20)]
        for k in range(20):
            pev[k][0].record(stream)
            mla.plan_device(shape, kvl0, ql0, plan_buf=dp.device, num_workgroups=nwg)
            pev[k][1].record(stream)
        torch.cuda.synchronize()
        plan_dev_us = sum(pev[k][0].elapsed_time(pev[k][1]) for k in range(20)) / 20 * 1e3
        log(f"device planner: avg {plan_dev_us:.2f} us")

    t_step = step_avg * 1e-3
    t_fwd = fwd_avg * 1e-3
    kv_gbs = kv_total / t_step / 1e9
    tflops = cnt["flops"] / t_step / 1e12
    t_hbm = cnt["alg_bytes"] / (HBM_PEAK_GBS * 1e9)
    t_mfma = cnt["flops"] / (MFMA_BF16_PEAK_TFLOPS * 1e12)
    if t_hbm >= t_mfma:
        achieved, peak, unit, bound = cnt["alg_bytes"] / t_fwd / 1e9, HBM_PEAK_GBS, "GB/s", "hbm"
    else:
        achieved, peak, unit, bound = cnt["flops"] / t_fwd / 1e12, MFMA_BF16_PEAK_TFLOPS, \
            "TFLOP/s", "mfma"
    kernel_name = decode_kernel_name(case.kv_dtype, pl.phases)
    kernel_sym = decode_kernel_symbol(case.kv_dtype, pl.phases)
    kernel_src = {W8_KERNEL: "decode_w8_kernel.hip", QRES_KERNEL: "decode_kernel_qres.hip",
                  SPLIT_KERNEL: "decode_split_kernel.hip"}.get(kernel_name, "decode_kernel.hip")
    traffic = read_traffic(args.workload, kernel_name, (kernel_src,), symbol=kernel_sym)

    res = {
        "metric": METRIC,
        "value": round(kv_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(step_avg, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if case.kv_dtype == "bf16" else "bf16+e4m3",
        "data": "synthetic",
        "config": {
            "workload": args.workload, "batch": case.batch, "num_heads": case.num_heads,
            "d_qk": case.d_qk, "d_v": case.d_latent, "q_len_max": case.max_q_len,
            "page_size": case.page_size, "kv_dtype": case.kv_dtype,
            "kv_tokens": int(full.kv_lens.astype("int64").sum()),
            "kv_len_mean": round(float(full.kv_lens.mean()), 1),
            "tree_drafts": tree is not None,
        },
        "us_per_call": round(step_avg * 1e3, 2),
        "us_fwd_kernel": round(fwd_avg * 1e3, 2),
        "us_per_call_pct": percentiles(step_ms),
        "us_fwd_kernel_pct": percentiles(fwd_ms),
        "us_per_call_warm": round(warm_avg * 1e3, 2),
        "us_per_call_graph": None if graph_avg is None else round(graph_avg * 1e3, 2),
        "us_tree_merge": None if tree_avg is None else round(tree_avg * 1e3, 2),
        "tflops": round(tflops, 2),
        "pct_roofline_call": round(100 * max(t_hbm, t_mfma) / t_step, 1),
        # the decode kernel's algorithmic MFMA work over its time, as a
        # fraction of the dense bf16 peak: a lower bound on the matrix units'
        # busy fraction (the kernel issues at least this work, more where a
        # key tile or a row block is padded), and the same for HBM bytes
        "mfma_frac_fwd": round(cnt["flops"] / t_fwd / (MFMA_BF16_PEAK_TFLOPS * 1e12), 4),
        "hbm_frac_fwd": round(cnt["alg_bytes"] / t_fwd / (HBM_PEAK_GBS * 1e9), 4),
        "roofline": {
            "bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4),
            "traffic": None if traffic is None else round(traffic),
            "kernel": kernel_name,
            "alg_bytes_per_launch": cnt["alg_bytes"], "flops_per_launch": cnt["flops"],
        },
        "plan": {"host_us": round(plan_us, 1),
                 "device_us": None if plan_dev_us is None else round(plan_dev_us, 1),
                 "workgroups": pl.info.num_workgroups,
                 "items": pl.info.num_items, "partials": pl.info.num_partials,
                 "combine_blocks": pl.info.num_combine},
        "wall_s_timed": round(wall, 4),
        "input_sets": nsets,
        "kernel_source_sha256": kernel_source_hash(),
        "code_object_sha256": code_object_hash(kernel_src, kernel_sym),
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log(f"cpu baseline: float64 oracle for about {args.cpu_seconds:.0f} s")
        seq_fn = None
        if tree is not None:
            from oracle import tree_ref
            seq_fn = lambda b: tree_ref.mla_decode_tree_ref_seq(full, tree, b)  # noqa: E731
        res["cpu_baseline"] = cpu_baseline(full, args.cpu_seconds, kv_total, seq_fn)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

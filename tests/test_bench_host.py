"""Host-side logic of bench.py (no GPU): the algorithmic byte and FLOP
counts behind the roofline fraction, the name of the kernel a plan launches,
and the counter summary lookup that goes stale when a kernel source changes."""
import math
import os

import numpy as np

import bench
from workloads import make_case


def test_workload_counts_by_hand():
    # two sequences, q_len 2 causal: visible keys per row are L-1 and L
    case = make_case(kv_lens=[100, 7], q_lens=[2, 1], num_heads=16, page_size=16, seed=3,
                     sm_scale=1 / math.sqrt(192))
    c = bench.workload_counts(case)
    assert c["kv_tokens"] == 107
    assert c["kv_bytes"] == 107 * 1152
    rows = (2 + 1) * 16
    pages = 7 + 1
    assert c["alg_bytes"] == 107 * 1152 + rows * (1152 + 1024 + 4) + pages * 4 + 2 * 8
    visible = (99 + 100) + 7
    assert c["flops"] == 2 * visible * 16 * (576 + 512)


def test_workload_counts_e4m3_row_bytes():
    case = make_case(kv_lens=[64], num_heads=16, kv_dtype="fp8_e4m3", seed=4,
                     sm_scale=1 / math.sqrt(192))
    assert bench.workload_counts(case)["kv_bytes"] == 64 * (576 + 4)


def test_decode_kernel_name_follows_the_plan():
    assert bench.decode_kernel_name("bf16", 1) == "mla_decode_kernel_pairs"
    assert bench.decode_kernel_name("bf16", 4) == "mla_decode_kernel"
    assert bench.decode_kernel_name("fp8_e4m3", 1) == "mla_decode_kernel"


def test_traffic_summary_keyed_by_source_hash(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    csrc = tmp_path / "mla_paged_decode_absorbed_amd" / "csrc"
    csrc.mkdir(parents=True)
    for name in bench.KERNEL_SOURCES:
        (csrc / name).write_text(name)
    h = bench.kernel_source_hash()
    f = prof / "mla_decode_kernel_pairs_wl_traffic.txt"
    f.write_text(f"# header\nkernel_source_sha256: {h}\nhbm_bytes_per_launch: 1234\n")
    assert bench.read_traffic("wl", "mla_decode_kernel_pairs") == 1234.0
    (csrc / bench.KERNEL_SOURCES[0]).write_text("changed")
    assert bench.read_traffic("wl", "mla_decode_kernel_pairs") is None
    assert bench.read_traffic("other", "mla_decode_kernel_pairs") is None

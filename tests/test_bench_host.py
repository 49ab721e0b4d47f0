"""Host-side logic of bench.py (no GPU): the algorithmic byte and FLOP
counts behind the roofline fraction, the name of the kernel a plan launches,
and the counter summary lookup that goes stale when a kernel source changes."""
import math
import os


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


def test_traffic_summary_keyed_by_code_object(tmp_path, monkeypatch):
    # a summary keyed by the machine code stays valid across source edits that
    # leave the code object alone, and goes stale when the code object changes
    import json
    prof = tmp_path / "profiles"
    prof.mkdir()
    build = tmp_path / "mla_paged_decode_absorbed_amd" / "_build"
    build.mkdir(parents=True)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    manifest = build / "code_objects.json"
    sym = bench.decode_kernel_symbol("bf16", 1)
    assert sym == "mla_decode_kernel_pairs<0>"
    manifest.write_text(json.dumps({"decode_kernel.hip": {sym: "00112233aabbccdd",
                                                          "other<1>": "1"}}))
    f = prof / "mla_decode_kernel_pairs_wl_traffic.txt"
    f.write_text("code_object_sha256: 00112233aabbccdd\nhbm_bytes_per_launch: 777\n")
    assert bench.read_traffic("wl", "mla_decode_kernel_pairs", symbol=sym) == 777.0
    # another kernel of the same file changing does not matter
    manifest.write_text(json.dumps({"decode_kernel.hip": {sym: "00112233aabbccdd",
                                                          "other<1>": "2"}}))
    assert bench.read_traffic("wl", "mla_decode_kernel_pairs", symbol=sym) == 777.0
    manifest.write_text(json.dumps({"decode_kernel.hip": {sym: "ffffffffffffffff"}}))
    assert bench.read_traffic("wl", "mla_decode_kernel_pairs", symbol=sym) is None
    manifest.unlink()
    assert bench.read_traffic("wl", "mla_decode_kernel_pairs", symbol=sym) is None


def test_percentiles_by_hand():
    p = bench.percentiles([0.001 * k for k in range(1, 12)])   # 1 .. 11 us
    assert p == {"p10": 2.0, "median": 6.0, "p90": 10.0}
    assert bench.percentiles([0.005]) == {"p10": 5.0, "median": 5.0, "p90": 5.0}


def test_build_manifest_matches_the_library_objects():
    # the manifest the build writes names every kernel source's code object
    import json
    from mla_paged_decode_absorbed_amd import build
    if not os.path.exists(build.CODE_OBJECTS):
        import pytest
        pytest.skip("library not built")
    with open(build.CODE_OBJECTS) as f:
        m = json.load(f)
    assert set(m) == {s for s in build.SOURCES if s.endswith(".hip")}
    for kvd in ("bf16", "fp8_e4m3"):
        for ph in (1, 2, 4):
            sym = bench.decode_kernel_symbol(kvd, ph)
            assert bench.code_object_hash("decode_kernel.hip", sym) == m["decode_kernel.hip"][sym]


def test_candidate_kernel_naming(monkeypatch):
    monkeypatch.setenv("MLA_DECODE_KERNEL", "w8")
    assert bench.decode_kernel_name("bf16", 1) == "mla_decode_kernel_w8"
    assert bench.decode_kernel_symbol("bf16", 1) == "mla_decode_kernel_w8<0>"
    assert bench.decode_kernel_name("fp8_e4m3", 1) == "mla_decode_kernel_w8"
    assert bench.decode_kernel_symbol("fp8_e4m3", 1) == "mla_decode_kernel_w8<1>"
    # plans the candidate does not cover (several phases) keep the library kernels
    assert bench.decode_kernel_name("bf16", 4) == "mla_decode_kernel"
    assert bench.decode_kernel_symbol("fp8_e4m3", 2) == "mla_decode_kernel<1, 2>"
    monkeypatch.setenv("MLA_DECODE_KERNEL", "qres")
    assert bench.decode_kernel_name("fp8_e4m3", 1) == "mla_decode_kernel_qres"
    assert bench.decode_kernel_symbol("fp8_e4m3", 1) == "mla_decode_kernel_qres<1, 1>"
    assert bench.decode_kernel_symbol("bf16", 1) == "mla_decode_kernel_pairs<0>"
    monkeypatch.setenv("MLA_DECODE_KERNEL", "split")
    assert bench.decode_kernel_name("bf16", 1) == "mla_decode_kernel_split"
    assert bench.decode_kernel_symbol("bf16", 1) == "mla_decode_kernel_split<0>"
    assert bench.decode_kernel_name("fp8_e4m3", 1) == "mla_decode_kernel_split"
    assert bench.decode_kernel_symbol("fp8_e4m3", 1) == "mla_decode_kernel_split<1>"
    # several phases keep the library kernels
    assert bench.decode_kernel_symbol("bf16", 2) == "mla_decode_kernel<0, 2>"
    monkeypatch.delenv("MLA_DECODE_KERNEL")
    assert bench.decode_kernel_symbol("bf16", 1) == "mla_decode_kernel_pairs<0>"

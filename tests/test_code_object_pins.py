"""The gfx950 machine code of the library's GPU kernels, pinned kernel by
kernel (CPU only: hipcc cross-compiles, nothing runs on a GPU).

Each kernel source is compiled device-only with the library's own flags; for
every kernel in its code object the test hashes the kernel's machine code
(its bytes of .text), its kernel descriptor (64 bytes of .rodata: register
counts, LDS and scratch sizes, launch properties; the field that locates the
code is masked, since adding another kernel to the file may move it) and its
entry of the code object metadata (argument layout, sizes).  The pinned
hashes are those of the build whose library passed the GPU parity, graph,
tree-draft and cache-append suites (and, for the prefill kernels, the
quantized-prefill suite) on MI355X.  A source edit that leaves the machine
code alone keeps the pins, and kernels may be added beside the pinned ones;
any change of a pinned kernel fails here, so no kernel that has not passed
the GPU suites replaces a validated one unnoticed.

The hashes hold for one compiler build only; under another one the test is
skipped (it says which).
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
from mla_paged_decode_absorbed_amd import build as libbuild  # noqa: E402

HIPCC = "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else shutil.which("hipcc")

# The compiler the pins were taken with.
PINNED_COMPILER = "AMD clang version 22.0.0git (https://github.com/RadeonOpenCompute/llvm-project " \
                  "roc-7.2.0 26014 7b800a19466229b8479a78de19143dc33c3ab9b5)"

# source -> {kernel (demangled name, template arguments kept): sha256 (16 hex
# digits) of its code, masked descriptor and metadata}
PINS = {
    "append_kernel.hip": {
        "mla_kv_append_kernel<0>": "af40742b52a854ed",
        "mla_kv_append_kernel<1>": "99a6f632625ccac8",
    },
    "combine_kernel.hip": {
        "mla_combine_kernel": "3b55ab76a3e9e923",
    },
    "decode_kernel.hip": {
        "mla_decode_kernel<0, 2>": "f68f1fafb811c729",
        "mla_decode_kernel<0, 4>": "f80e603336080f50",
        "mla_decode_kernel<1, 1>": "4561acbbca3d28d9",
        "mla_decode_kernel<1, 2>": "12030241895c4f29",
        "mla_decode_kernel<1, 4>": "1385b15ad6d2f593",
        "mla_decode_kernel_pairs<0>": "01606bf0968b13e5",
    },
    "plan_kernel.hip": {
        "mla_plan_kernel": "37c084122812ee11",
    },
    "prefill_attn_kernel.hip": {
        "mla_prefill_attn_kernel<4, 1>": "6134ed22eb397dcc",
    },
    "prefill_quant_kernel.hip": {
        "mla_prefill_quant_k_kernel": "e9418dd04c1a1462",
        "mla_prefill_quant_q_kernel": "d7c6220d5a7f9bef",
        "mla_prefill_quant_v_kernel": "0c5fed5eae148b9b",
    },
    "tree_kernel.hip": {
        "mla_tree_kernel": "925d7d16b9f574d5",
    },
}

# Kernel sources added after the last GPU run of this library; none of them is
# on the default decode path.
NOT_YET_RUN_ON_GPU = (
    "check_kernel.hip",       # mla_decode_check, opt-in debug mode
    "decode_w8_kernel.hip",   # two-waves-per-SIMD candidate, only under MLA_DECODE_KERNEL=w8
    "decode_kernel_qres.hip", # e4m3 kernels with Q resident, only under MLA_DECODE_KERNEL=qres
    "decode_split_kernel.hip",  # pairs of waves sharing 32 rows, only under MLA_DECODE_KERNEL=split
)
# Kernels added since to a pinned source, beside its validated kernels; none
# of them is on the default path either.
NEW_KERNELS_IN_PINNED_SOURCES = {
    "combine_kernel.hip": {"mla_combine_kernel_bf16"},   # merge of the candidate's bf16 partials
}

pytestmark = pytest.mark.skipif(HIPCC is None, reason="ROCm toolchain not available")


def _compiler_id() -> str:
    res = subprocess.run([HIPCC, "--version"], capture_output=True, text=True)
    for line in res.stdout.splitlines():
        if line.startswith("AMD clang version"):
            return line.strip()
    return ""


# The fingerprint (code bytes, masked descriptor, metadata entry) is
# libbuild.kernel_fingerprints; the planted-change test below checks that it
# sees a one-byte change of one kernel and nothing of its neighbour.
kernel_fingerprints = libbuild.kernel_fingerprints


def compile_code_object(src: str, workdir: str) -> str:
    co = os.path.join(workdir, src + ".co")
    cmd = [HIPCC, *libbuild.common_flags(), "--cuda-device-only", "--no-gpu-bundle-output",
           "-c", os.path.join(libbuild.CSRC, src), "-o", co]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    return co


@pytest.fixture(scope="module")
def fingerprints(tmp_path_factory):
    if _compiler_id() != PINNED_COMPILER:
        pytest.skip(f"pins were taken with {PINNED_COMPILER!r}, this is {_compiler_id()!r}")
    pytest.importorskip("msgpack")
    d = str(tmp_path_factory.mktemp("co"))
    with ThreadPoolExecutor(max_workers=4) as ex:
        cos = list(ex.map(lambda s: compile_code_object(s, d), sorted(PINS)))
    return {src: kernel_fingerprints(co) for src, co in zip(sorted(PINS), cos)}


@pytest.mark.parametrize("src", sorted(PINS))
def test_validated_kernels_are_unchanged(fingerprints, src):
    got = fingerprints[src]
    for kernel, pin in PINS[src].items():
        assert kernel in got, f"{src}: validated kernel {kernel} is gone ({sorted(got)})"
        assert got[kernel] == pin, (
            f"{src}: {kernel} changed ({got[kernel]} != pinned {pin}); code that has not "
            "passed the GPU suites must not replace a validated kernel")


@pytest.mark.parametrize("src", sorted(PINS))
def test_every_kernel_of_a_pinned_source_is_pinned_or_new(fingerprints, src):
    extra = set(fingerprints[src]) - set(PINS[src])
    assert extra == NEW_KERNELS_IN_PINNED_SOURCES.get(src, set()), (src, sorted(extra))


def test_every_library_kernel_source_is_pinned_or_new():
    """Every HIP source of the library is either pinned here or listed as a
    kernel source added since, whose GPU status the design notes state."""
    srcs = {s for s in libbuild.SOURCES if s.endswith(".hip")}
    unpinned = srcs - set(PINS)
    assert unpinned <= set(NOT_YET_RUN_ON_GPU), sorted(unpinned - set(NOT_YET_RUN_ON_GPU))


def test_fingerprint_sees_a_one_byte_change(tmp_path):
    """A planted change of one instruction byte of one kernel changes that
    kernel's fingerprint and not its neighbour's."""
    if _compiler_id() != PINNED_COMPILER:
        pytest.skip("other compiler")
    pytest.importorskip("msgpack")
    co = compile_code_object("append_kernel.hip", str(tmp_path))
    before = kernel_fingerprints(co)
    with open(co, "rb") as f:
        blob = bytearray(f.read())
    secs, cstr = libbuild._elf_sections(bytes(blob))
    syms = libbuild._elf_symbols(bytes(blob), secs, cstr)
    kd = next(md[".symbol"] for md in libbuild._amdgpu_kernels_metadata(bytes(blob), secs)
              if libbuild.kernel_short_name(md[".name"]) == "mla_kv_append_kernel<1>")
    value, size, shndx = syms[kd[:-3]]
    pos = secs[shndx]["off"] + value - secs[shndx]["addr"] + size // 2
    blob[pos] ^= 0x01
    planted = tmp_path / "planted.co"
    planted.write_bytes(bytes(blob))
    after = kernel_fingerprints(str(planted))
    assert after["mla_kv_append_kernel<1>"] != before["mla_kv_append_kernel<1>"]
    assert after["mla_kv_append_kernel<0>"] == before["mla_kv_append_kernel<0>"]


def test_short_names():
    assert libbuild.kernel_short_name(
        "_ZN3mla12_GLOBAL__N_117mla_decode_kernelILi1ELi4EEEvNS_10DecodeArgsE") == \
        "mla_decode_kernel<1, 4>"
    assert libbuild.kernel_short_name(
        "_ZN3mla12_GLOBAL__N_118mla_combine_kernelENS_11CombineArgsE") == "mla_combine_kernel"

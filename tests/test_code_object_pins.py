"""The gfx950 machine code of the library's GPU kernels, pinned (CPU only:
hipcc cross-compiles, nothing runs on a GPU).

Each kernel source is compiled device-only with the library's own flags, and
the code object's machine code (.text), kernel descriptors (.rodata: register
counts, LDS size, launch properties) and metadata (.note) are hashed.  The
pinned hashes are those of the build whose library passed the GPU parity,
graph-replay, tree-draft and cache-append suites (and, for the prefill
kernels, the quantized-prefill suite) on MI355X.  A source edit that leaves
the machine code alone keeps the pin; any change of the code that runs on
the GPU fails here, so it cannot enter the library unnoticed.

The hashes hold for one compiler build only; under another one the test is
skipped (it says which).
"""
import hashlib
import os
import re
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
from mla_paged_decode_absorbed_amd import build as libbuild  # noqa: E402

LLVM = "/opt/rocm/llvm/bin"
HIPCC = "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else shutil.which("hipcc")

# The compiler the pins were taken with.
PINNED_COMPILER = "AMD clang version 22.0.0git (https://github.com/RadeonOpenCompute/llvm-project " \
                  "roc-7.2.0 26014 7b800a19466229b8479a78de19143dc33c3ab9b5)"

# sha256 (first 16 hex digits) of .text + .rodata + .note of each source's
# gfx950 code object.
PINS = {
    "decode_kernel.hip": "2f71c036ab578aff",
    "combine_kernel.hip": "95b0acb3adf772a6",
    "append_kernel.hip": "845cbeead2be0fec",
    "plan_kernel.hip": "7b64942843243e1d",
    "tree_kernel.hip": "1342ea6d494bdfca",
    "prefill_quant_kernel.hip": "f3ac478ecf16a5f1",
    "prefill_attn_kernel.hip": "181cb571a4592cb5",
}

pytestmark = pytest.mark.skipif(
    HIPCC is None or not os.path.exists(os.path.join(LLVM, "llvm-objcopy")),
    reason="ROCm toolchain not available")


def _compiler_id() -> str:
    res = subprocess.run([HIPCC, "--version"], capture_output=True, text=True)
    for line in res.stdout.splitlines():
        if line.startswith("AMD clang version"):
            return line.strip()
    return ""


def code_object_hash(src: str, workdir: str) -> str:
    """Hash of the gfx950 code object that the library build embeds for one
    source file (same flags; device-only, unbundled)."""
    co = os.path.join(workdir, src + ".co")
    cmd = [HIPCC, *libbuild.common_flags(), "--cuda-device-only", "--no-gpu-bundle-output",
           "-c", os.path.join(libbuild.CSRC, src), "-o", co]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    h = hashlib.sha256()
    for sec in (".text", ".rodata", ".note"):
        out = os.path.join(workdir, f"{src}{sec}.bin")
        res = subprocess.run([os.path.join(LLVM, "llvm-objcopy"), "-O", "binary",
                              f"--only-section={sec}", co, out], capture_output=True, text=True)
        assert res.returncode == 0, res.stderr
        with open(out, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


@pytest.fixture(scope="module")
def hashes(tmp_path_factory):
    if _compiler_id() != PINNED_COMPILER:
        pytest.skip(f"pins were taken with {PINNED_COMPILER!r}, this is {_compiler_id()!r}")
    d = str(tmp_path_factory.mktemp("co"))
    with ThreadPoolExecutor(max_workers=4) as ex:
        vals = list(ex.map(lambda s: code_object_hash(s, d), sorted(PINS)))
    return dict(zip(sorted(PINS), vals))


@pytest.mark.parametrize("src", sorted(PINS))
def test_kernel_machine_code_is_the_validated_one(hashes, src):
    assert hashes[src] == PINS[src], (
        f"{src}: the gfx950 code object changed ({hashes[src]} != pinned {PINS[src]}); "
        "code that has not passed the GPU suites must not replace the validated kernels")


def test_every_library_kernel_source_is_pinned_or_new():
    """Every HIP source of the library is either pinned here or listed as a
    kernel added since, whose GPU status the design notes state."""
    srcs = {s for s in libbuild.SOURCES if s.endswith(".hip")}
    unpinned = srcs - set(PINS)
    assert unpinned <= set(NOT_YET_RUN_ON_GPU), sorted(unpinned - set(NOT_YET_RUN_ON_GPU))
    assert not re.search(r"\s", "".join(srcs))


# Kernel sources added after the last GPU run of this library; none of them is
# on the default decode path.
NOT_YET_RUN_ON_GPU = ("check_kernel.hip",)   # mla_decode_check, opt-in debug mode

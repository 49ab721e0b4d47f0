"""Build libmla_decode.so (gfx950) in-tree with hipcc.

Usage: python -m mla_paged_decode_absorbed_amd.build [--jobs N]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libmla_decode.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
OBJ_DIR = os.path.join(PKG, "_build")
# sha256 (16 hex digits) of each kernel source's gfx950 code object (.text,
# .rodata, .note), written by build(): profiles keyed by it stay valid across
# source edits that leave the machine code alone
CODE_OBJECTS = os.path.join(OBJ_DIR, "code_objects.json")
LLVM_BIN = "/opt/rocm/llvm/bin"

SOURCES = ["api.cpp", "plan.cpp", "decode_kernel.hip", "combine_kernel.hip", "append_kernel.hip",
           "plan_kernel.hip", "tree_kernel.hip", "prefill_quant_kernel.hip",
           "prefill_attn_kernel.hip", "check_kernel.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required)")


def common_flags() -> list[str]:
    return [
        "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
        f"-I{INCLUDE}", f"-I{CSRC}",
        # keep the compiler from forming packed-fp32 VALU ops
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-unused-command-line-argument",
    ]


def _compile(src: str) -> str:
    obj = os.path.join(OBJ_DIR, src + ".o")
    cmd = [hipcc(), *common_flags(), "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def code_object_hash(obj: str) -> str | None:
    """Hash of the gfx950 code object embedded in a hipcc object file, or None
    if the LLVM tools are missing."""
    objcopy = os.path.join(LLVM_BIN, "llvm-objcopy")
    bundler = os.path.join(LLVM_BIN, "clang-offload-bundler")
    if not (os.path.exists(objcopy) and os.path.exists(bundler)):
        return None
    with tempfile.TemporaryDirectory() as d:
        fat, co = os.path.join(d, "fat"), os.path.join(d, "co")
        steps = [[objcopy, f"--dump-section=.hip_fatbin={fat}", obj, os.path.join(d, "o")],
                 [bundler, "--unbundle", "--type=o", f"--input={fat}",
                  f"--targets=hipv4-amdgcn-amd-amdhsa--{ARCH}", f"--output={co}"]]
        for cmd in steps:
            if subprocess.run(cmd, capture_output=True).returncode != 0:
                return None
        h = hashlib.sha256()
        for sec in (".text", ".rodata", ".note"):
            out = os.path.join(d, sec)
            if subprocess.run([objcopy, "-O", "binary", f"--only-section={sec}", co, out],
                              capture_output=True).returncode != 0:
                return None
            with open(out, "rb") as f:
                h.update(f.read())
    return h.hexdigest()[:16]


def build(jobs: int = 4, verbose: bool = False) -> str:
    """Compile every source for gfx950 and link the shared library."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    manifest = {}
    for src, obj in zip(SOURCES, objs):
        if src.endswith(".hip"):
            manifest[src] = code_object_hash(obj)
    with open(CODE_OBJECTS, "w") as f:
        json.dump(manifest, f, indent=1, sort_keys=True)
    if verbose:
        print(f"built {LIB_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=4)
    args = ap.parse_args()
    build(args.jobs, verbose=True)
    sys.exit(0)

"""Build libmla_decode.so (gfx950) in-tree with hipcc.

Usage: python -m mla_paged_decode_absorbed_amd.build [--jobs N]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import shutil
import struct
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
# {source: {kernel: fingerprint}} of the built gfx950 code objects (see
# kernel_fingerprints), written by build(): profiles keyed by a kernel's
# fingerprint stay valid across source edits that leave its machine code alone
CODE_OBJECTS = os.path.join(OBJ_DIR, "code_objects.json")
LLVM_BIN = "/opt/rocm/llvm/bin"

SOURCES = ["api.cpp", "plan.cpp", "decode_kernel.hip", "combine_kernel.hip", "append_kernel.hip",
           "plan_kernel.hip", "tree_kernel.hip", "prefill_quant_kernel.hip",
           "prefill_attn_kernel.hip", "check_kernel.hip", "decode_w8_kernel.hip",
           "decode_kernel_qres.hip", "decode_split_kernel.hip"]
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


def _elf_sections(blob: bytes):
    shoff, = struct.unpack_from("<Q", blob, 0x28)
    shentsize, shnum, shstrndx = struct.unpack_from("<HHH", blob, 0x3A)
    secs = []
    for i in range(shnum):
        name, typ, _fl, addr, off, size, link, _inf, _al, entsize = struct.unpack_from(
            "<IIQQQQIIQQ", blob, shoff + i * shentsize)
        secs.append(dict(name=name, addr=addr, off=off, size=size, link=link, entsize=entsize))

    def cstr(sec, o):
        start = sec["off"] + o
        return blob[start:blob.index(b"\0", start)].decode()

    for sec in secs:
        sec["sname"] = cstr(secs[shstrndx], sec["name"])
    return secs, cstr


def _elf_symbols(blob: bytes, secs, cstr):
    out = {}
    for sec in secs:
        if sec["sname"] != ".symtab":
            continue
        for k in range(sec["size"] // sec["entsize"]):
            name, _info, _other, shndx, value, size = struct.unpack_from(
                "<IBBHQQ", blob, sec["off"] + k * sec["entsize"])
            if name:
                out[cstr(secs[sec["link"]], name)] = (value, size, shndx)
    return out


def _amdgpu_kernels_metadata(blob: bytes, secs):
    import msgpack
    note = next(sec for sec in secs if sec["sname"] == ".note")
    off, end = note["off"], note["off"] + note["size"]
    while off < end:
        namesz, descsz, typ = struct.unpack_from("<III", blob, off)
        name = blob[off + 12: off + 12 + namesz].rstrip(b"\0")
        dstart = off + 12 + (namesz + 3) // 4 * 4
        if name == b"AMDGPU" and typ == 32:   # NT_AMDGPU_METADATA (msgpack)
            return msgpack.unpackb(blob[dstart: dstart + descsz], raw=False)["amdhsa.kernels"]
        off = dstart + (descsz + 3) // 4 * 4
    raise ValueError("no AMDGPU metadata note")


def kernel_short_name(mangled: str) -> str:
    """Kernel name with its integer template arguments, from the mangled
    symbol: '_ZN3mla12_GLOBAL__N_117mla_decode_kernelILi1ELi4EEEv...' ->
    'mla_decode_kernel<1, 4>'."""
    for m in re.finditer(r"\d+", mangled):
        digits, end = m.group(0), m.end()
        for k in range(len(digits)):   # '117mla_...' after '_N_1' is length 17
            n = int(digits[k:])
            ident = mangled[end:end + n]
            if len(ident) == n and ident.startswith("mla_") and re.fullmatch(r"\w+", ident):
                args = re.match(r"I((?:Li-?\d+E)+)E", mangled[end + n:])
                if args:
                    vals = re.findall(r"Li(-?\d+)E", args.group(1))
                    return f"{ident}<{', '.join(vals)}>"
                return ident
    return mangled


def kernel_fingerprints(co_path: str) -> dict:
    """{kernel: sha256 (16 hex digits)} for every kernel of a gfx950 code
    object: its machine code, its 64-byte kernel descriptor with the field
    that locates the code masked (another kernel in the file may move it),
    and its metadata entry (argument layout, register and LDS sizes)."""
    with open(co_path, "rb") as f:
        blob = f.read()
    secs, cstr = _elf_sections(blob)
    syms = _elf_symbols(blob, secs, cstr)
    out = {}
    for md in _amdgpu_kernels_metadata(blob, secs):
        kd_sym = md[".symbol"]
        value, size, shndx = syms[kd_sym[:-3] if kd_sym.endswith(".kd") else kd_sym]
        text = secs[shndx]
        code = blob[text["off"] + value - text["addr"]: text["off"] + value - text["addr"] + size]
        kv, ks, kidx = syms[kd_sym]
        ro = secs[kidx]
        kd = bytearray(blob[ro["off"] + kv - ro["addr"]: ro["off"] + kv - ro["addr"] + ks])
        kd[16:24] = bytes(8)   # kernel_code_entry_byte_offset
        h = hashlib.sha256()
        h.update(code)
        h.update(bytes(kd))
        h.update(json.dumps(md, sort_keys=True, default=str).encode())
        out[kernel_short_name(md[".name"])] = h.hexdigest()[:16]
    return out


def object_fingerprints(obj: str) -> dict | None:
    """kernel_fingerprints of the gfx950 code object embedded in a hipcc
    object file, or None if the LLVM tools or msgpack are missing."""
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
        try:
            return kernel_fingerprints(co)
        except (ImportError, ValueError, KeyError):
            return None


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
            manifest[src] = object_fingerprints(obj)
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

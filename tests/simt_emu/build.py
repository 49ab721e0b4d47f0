"""Build tests/simt_emu/_build/run_case: the library's kernel sources compiled
for the host CPU against the lane-thread emulator, with AddressSanitizer.

The kernel sources are copied unchanged next to the emulator's version of
gfx950_asm.h (the only file replaced), so the emulated code is the code the
gfx950 library is built from.  Host-only: nothing here targets a GPU.
"""
from __future__ import annotations

import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
CSRC = os.path.join(ROOT, "mla_paged_decode_absorbed_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(HERE, "_build")
BIN = os.path.join(OUT, "run_case")

KERNEL_FILES = ["decode_kernel.hip", "combine_kernel.hip", "append_kernel.hip",
                "plan_kernel.hip", "tree_kernel.hip", "api.cpp", "plan.cpp", "kernels.h",
                "append.h", "plan_core.h", "plan_device.h", "tree.h", "plan_layout.h",
                "validate.h", "prefill.h", "prefill_quant_kernel.hip", "prefill_attn_kernel.hip",
                "check.h", "check_kernel.hip", "decode_w8_kernel.hip", "decode_kernel_qres.hip",
                "decode_split_kernel.hip"]


# compilation units of the library built into the emulator binary
UNITS = ("decode_kernel.hip", "combine_kernel.hip", "append_kernel.hip", "plan_kernel.hip",
         "tree_kernel.hip", "prefill_quant_kernel.hip", "prefill_attn_kernel.hip",
         "check_kernel.hip", "decode_w8_kernel.hip", "decode_kernel_qres.hip",
         "decode_split_kernel.hip", "api.cpp", "plan.cpp")


def _includes(path: str, src: str, seen=None) -> set:
    """Local headers a source includes, directly or through other local
    headers (#include "name" found in src)."""
    import re
    seen = set() if seen is None else seen
    for name in re.findall(r'^\s*#include\s+"([^"]+)"', open(path).read(), re.M):
        h = os.path.join(src, name)
        if name not in seen and os.path.exists(h):
            seen.add(name)
            _includes(h, src, seen)
    return seen


def compiler() -> str:
    for c in ("/opt/rocm/llvm/bin/clang++", shutil.which("clang++")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("clang++ not found")


def build(sanitize: bool = True, decode_source: str | None = None, tag: str = "",
          patches: dict | None = None, ubsan: bool = False, lds_trace: bool = False) -> str:
    """Build the emulator binary.  ``decode_source`` replaces the library's
    decode_kernel.hip (a candidate kernel); ``patches`` maps a copied source
    file to (old, new) text replacements, each of which must apply (a variant
    of the library, built on the CPU only); ``tag`` names that binary;
    ``ubsan`` adds UndefinedBehaviorSanitizer (every unit rebuilt, the run
    stopping at the first report); ``lds_trace`` makes the decode kernels'
    LDS pointers log their accesses for the bank model (every unit rebuilt;
    the counts are written where EMU_LDS_STATS names) and for the race
    detector (run with EMU_LDS_RACE set)."""
    out = os.path.join(OUT, tag) if tag else OUT
    src = os.path.join(out, "src")
    os.makedirs(src, exist_ok=True)
    for f in KERNEL_FILES:
        shutil.copyfile(os.path.join(CSRC, f), os.path.join(src, f))
    if decode_source:
        shutil.copyfile(decode_source, os.path.join(src, "decode_kernel.hip"))
    for fname, reps in (patches or {}).items():
        path = os.path.join(src, fname)
        text = open(path).read()
        for old, new in reps:
            if text.count(old) != 1:
                raise RuntimeError(f"patch for {fname} does not apply once: {old!r}")
            text = text.replace(old, new)
        with open(path, "w") as fh:
            fh.write(text)
    shutil.copyfile(os.path.join(HERE, "gfx950_asm.h"), os.path.join(src, "gfx950_asm.h"))
    # -O2 (EMU_OPT overrides): AddressSanitizer checks every memory access the
    # optimised code still makes (the planted out-of-bounds cases fail as at
    # -O1), and the emulation runs about 1.5 times faster
    flags = ["-std=c++20", os.environ.get("EMU_OPT", "-O2"), "-g", "-pthread", "-fno-omit-frame-pointer",
             f"-I{HERE}", f"-I{src}", f"-I{INCLUDE}", "-Wno-unused-command-line-argument", "-Wno-psabi"]
    if sanitize:
        flags.append("-fsanitize=address")
    if ubsan:
        flags += ["-fsanitize=undefined", "-fno-sanitize-recover=undefined"]
    if lds_trace:
        flags.append("-DEMU_LDS_TRACE")
    units = [os.path.join(src, f) for f in UNITS]
    units += [os.path.join(HERE, "emu_runtime.cpp"), os.path.join(HERE, "run_case.cpp")]
    # A variant recompiles only the units that are, or include, a changed
    # file, and links the other objects of its base build (the default one,
    # or the LDS-trace one for a traced variant), brought up to date first.
    changed = set(patches or {}) | ({"decode_kernel.hip"} if decode_source else set())
    reuse = bool(tag) and sanitize and not ubsan and tag != TRACE_TAG
    base = os.path.join(OUT, TRACE_TAG) if lds_trace else OUT
    if reuse and lds_trace:
        trace_binary()
    elif reuse:
        from tests.simt_emu import harness as _h
        _h.ensure_built()

    def compile_unit(u):
        name = os.path.basename(u)
        if reuse and not (_includes(u, src) & changed) and name not in changed:
            return os.path.join(base, name + ".o")
        obj = os.path.join(out, name + ".o")
        cmd = [compiler(), *flags, "-x", "c++", "-c", u, "-o", obj]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"emulator build failed on {u}:\n{res.stderr[-4000:]}")
        return obj

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_unit, units))
    binary = os.path.join(out, "run_case")
    cmd = [compiler(), *flags, *objs, "-o", binary]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"emulator link failed:\n{res.stderr[-4000:]}")
    return binary


TRACE_TAG = "ldstrace"


def fresh_build(tag: str, **kw) -> str:
    """build(tag=tag, **kw) unless that binary exists and is newer than every
    source (for builds without patches: their options are fixed by the tag).
    Not safe to call from several threads while the binary is stale."""
    from tests.simt_emu import harness as _h
    if kw.get("patches") or kw.get("decode_source"):
        raise ValueError("fresh_build is for builds without patches")
    path = os.path.join(OUT, tag, "run_case")
    if not os.path.exists(path) or _h._stale(path):
        build(tag=tag, **kw)
    return path


def trace_binary() -> str:
    """The LDS-trace build (bank model and race detector), the base that
    traced variants link against."""
    return fresh_build(TRACE_TAG, lds_trace=True)


def build_exhaustive() -> str:
    """Host binary of append_exhaustive.cpp (the cache-append kernel's
    arithmetic checked over all inputs), optimized; linked with the emulator
    runtime, which needs the AddressSanitizer fiber interface."""
    out = os.path.join(OUT, "exhaustive")
    src = os.path.join(out, "src")
    os.makedirs(src, exist_ok=True)
    for f in KERNEL_FILES:
        shutil.copyfile(os.path.join(CSRC, f), os.path.join(src, f))
    shutil.copyfile(os.path.join(HERE, "gfx950_asm.h"), os.path.join(src, "gfx950_asm.h"))
    flags = ["-std=c++20", "-O2", "-pthread", "-ffp-contract=off", "-fsanitize=address",
             f"-I{HERE}", f"-I{src}", f"-I{INCLUDE}", "-Wno-unused-command-line-argument",
             "-Wno-psabi"]
    binary = os.path.join(out, "append_exhaustive")
    cmd = [compiler(), *flags, "-x", "c++", os.path.join(HERE, "append_exhaustive.cpp"),
           "-x", "c++", os.path.join(HERE, "emu_runtime.cpp"), "-o", binary]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"exhaustive check build failed:\n{res.stderr[-4000:]}")
    return binary


if __name__ == "__main__":
    print(build())

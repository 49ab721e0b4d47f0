"""Build the GPU check libraries of tests/gpu_checks in-tree (gfx950).

Test infrastructure only: each library holds one checking or measuring
kernel that a ``-m gpu`` test loads with ctypes.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CHECKS = {"e4m3_convert_check.hip": "libe4m3_convert_check.so",
          "lds_read_probe.hip": "liblds_read_probe.so"}


def build(verbose: bool = False) -> list[str]:
    from mla_paged_decode_absorbed_amd.build import ARCH, common_flags, hipcc

    out = []
    for src, lib in CHECKS.items():
        path = os.path.join(HERE, lib)
        cmd = [hipcc(), *common_flags(), "-shared", os.path.join(HERE, src), "-o", path + ".tmp"]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src} ({ARCH}):\n{res.stderr[-3000:]}")
        os.replace(path + ".tmp", path)
        if verbose:
            print(f"built {path}")
        out.append(path)
    return out


if __name__ == "__main__":
    build(verbose=True)

"""Runs bench.py's main() on the CPU with the GPU stubbed out (test helper).

torch.cuda (events, streams, graphs, device placement) and the library's
launching calls are replaced by stand-ins, so every Python path of bench.py
(argument handling, workload generation, planning through the real host
planner, timing arithmetic, roofline and JSON assembly, the oracle baseline)
runs without a GPU and without launching anything; the numbers it prints are
meaningless, the shape of its output is what is checked.  Used by
tests/test_bench_stub.py in a subprocess, since the stand-ins patch torch for
the whole process.

usage: python tests/bench_stub_run.py <bench.py arguments>
"""
import contextlib
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import torch  # noqa: E402

import mla_paged_decode_absorbed_amd as mla  # noqa: E402


class _Event:
    clock = 0.0

    def __init__(self, enable_timing=True):
        self.t = 0.0

    def record(self, stream=None):
        _Event.clock += 0.1
        self.t = _Event.clock

    def elapsed_time(self, other):
        return other.t - self.t


class _Stream:
    cuda_stream = 0


class _Graph:
    def replay(self):
        pass


def _strip_device(f):
    def g(*a, **k):
        k.pop("device", None)
        return f(*a, **k)
    return g


def install():
    torch.cuda.is_available = lambda: True
    torch.cuda.set_device = lambda d: None
    torch.cuda.synchronize = lambda *a: None
    torch.cuda.current_stream = lambda *a: _Stream()
    torch.cuda.Event = _Event
    torch.cuda.CUDAGraph = _Graph
    torch.cuda.graph = lambda g, **k: contextlib.nullcontext()
    to = torch.Tensor.to

    def to_host(self, *a, **k):
        if a and (str(a[0]).startswith("cuda") or isinstance(a[0], torch.device)):
            return self.clone()
        k.pop("device", None)
        return to(self, *a, **k) if a or k else self

    torch.Tensor.to = to_host
    torch.empty, torch.full, torch.ones = (_strip_device(torch.empty), _strip_device(torch.full),
                                           _strip_device(torch.ones))
    torch.zeros = _strip_device(torch.zeros)
    torch.empty_like = _strip_device(torch.empty_like)
    for name in ("decode_fwd", "combine", "tree_attend", "kv_append", "prefill_quantize",
                 "prefill_attn"):
        setattr(mla, name, lambda *a, **k: None)
    mla.plan_device = lambda shape, kvl, ql=None, **k: mla.plan(
        shape, kvl.numpy(), None if ql is None else ql.numpy(), upload=False,
        num_workgroups=k.get("num_workgroups") or 256, fixed=True)
    mla.load_library().mla_device_num_cus = lambda d: 256


if __name__ == "__main__":
    install()
    import bench
    sys.argv = ["bench.py"] + sys.argv[1:]
    sys.exit(bench.main())

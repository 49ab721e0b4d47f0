"""LDS read throughput per CU on MI355X, for the two read forms the decode
kernels use (16-byte ds_read_b128 for key fragments, ds_read_b64_tr_b16 for
transposed value fragments) with four and with eight waves per workgroup, one
workgroup per CU (tests/gpu_checks/lds_read_probe.hip).  A measurement, not a
parity test: it prints bytes per clock per CU (at the 2.4 GHz peak engine
clock) and checks only that the figures are plausible.  The figure bounds how
busy a decode kernel with two waves per SIMD can keep its matrix units.
Skipped, like the candidate kernels' tests, until its first GPU run.  (Named
to run after every validated suite.)"""
import ctypes
import os

import pytest

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(os.environ.get("MLA_RUN_UNVALIDATED") != "1",
                       reason="probe kernel not yet run on a GPU: set MLA_RUN_UNVALIDATED=1 "
                              "for its first run"),
]

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "gpu_checks",
                   "liblds_read_probe.so")
CLOCK_HZ = 2.4e9
GRID = 256   # one workgroup per CU


def _lib():
    if not os.path.exists(LIB):
        raise RuntimeError(f"{LIB} is missing: run __graft_entry__.build()")
    lib = ctypes.CDLL(LIB)
    lib.lds_read_probe.restype = ctypes.c_int
    lib.lds_read_probe.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_void_p, ctypes.c_void_p]
    return lib


@pytest.mark.parametrize("mode,width", [(0, 1024), (1, 512)])
@pytest.mark.parametrize("waves", [4, 8])
def test_lds_read_throughput(mode, width, waves):
    lib = _lib()
    out = torch.zeros(GRID * waves * 64, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    iters = 2048
    assert lib.lds_read_probe(waves, mode, 16, GRID, out.data_ptr(), stream.cuda_stream) == 0
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    assert lib.lds_read_probe(waves, mode, iters, GRID, out.data_ptr(), stream.cuda_stream) == 0
    t1.record(stream)
    torch.cuda.synchronize()
    sec = t0.elapsed_time(t1) * 1e-3
    per_cu = waves * iters * 8 * width              # bytes one workgroup reads
    b_per_clk = per_cu / sec / CLOCK_HZ
    form = "ds_read_b128" if mode == 0 else "ds_read_b64_tr_b16"
    print(f"LDS {form}, {waves} waves per CU: {b_per_clk:.1f} B/clock/CU at 2.4 GHz "
          f"({per_cu / sec / 1e9:.1f} GB/s per CU, {sec * 1e6:.1f} us)", flush=True)
    assert 1.0 < b_per_clk < 4096.0

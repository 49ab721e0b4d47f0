"""GPU parity of the library's e4m3 decode kernels rebuilt with the query
fragments resident before the key loop (decode_kernel_qres.hip, selected by
MLA_DECODE_KERNEL=qres for e4m3 caches) against the float64 oracle, at the
fp8 bars.

The rebuild has passed the CPU emulator and the machine-code checks
(tests/test_kernel_emulated.py, tests/test_kernel_isa.py) but has not run on a
GPU yet, so these cases are skipped unless MLA_RUN_UNVALIDATED=1 asks for its
first GPU run.  (Named to run after every validated suite.)"""
import math
import os

import pytest

from workloads import make_case, workload

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(os.environ.get("MLA_RUN_UNVALIDATED") != "1",
                       reason="rebuilt kernels not yet run on a GPU: set MLA_RUN_UNVALIDATED=1 "
                              "for their first run"),
]

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from tests.test_gpu_parity import check, run_gpu  # noqa: E402


@pytest.fixture(autouse=True)
def qres(monkeypatch):
    monkeypatch.setenv("MLA_DECODE_KERNEL", "qres")


@pytest.mark.parametrize("kv_lens,q_lens,nwg,phases", [
    ([1, 15, 16, 17, 129, 31, 33], [1, 1, 2, 1, 2, 1, 2], 12, 1),
    ([3000, 700, 65, 1800], [1, 2, 1, 2], 1, 1),
    ([3000, 700, 65, 1800], [1, 2, 1, 2], 256, 1),
    ([900, 70], [1, 2], 16, 4),
    ([700, 130, 5], [2, 2, 1], 8, 2),
])
def test_qres_small_cases(kv_lens, q_lens, nwg, phases):
    case = make_case(kv_lens=kv_lens, q_lens=q_lens, seed=29, max_q_len=2, kv_dtype="fp8_e4m3",
                     sm_scale=1 / math.sqrt(192))
    print(f"qres: lengths {kv_lens} q {q_lens} workgroups {nwg} phases {phases}", flush=True)
    (out, lse), pl = run_gpu(case, num_workgroups=nwg, phases=phases)
    assert pl.phases == phases
    check(case, out, lse)


def test_qres_long_context():
    case = workload("long_ctx_fp8")
    print("qres: long_ctx_fp8 (every sequence)", flush=True)
    (out, lse), _ = run_gpu(case)
    worst, rel = check(case, out, lse)
    print(f"qres: long_ctx_fp8: max-abs {worst:.3g} rel-L2 {rel:.3g}", flush=True)

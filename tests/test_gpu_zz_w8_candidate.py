"""GPU parity of the two-waves-per-SIMD candidate decode kernel
(decode_w8_kernel.hip, selected by MLA_DECODE_KERNEL=w8 for one-phase plans,
bf16 or e4m3 cache) against the float64 oracle, at the decode bars.

The candidate has passed the CPU emulator (both copy-landing modes and the
drift schedule, tests/test_kernel_emulated.py) and the machine-code checks
(tests/test_kernel_isa.py) but has not run on a GPU yet, so these cases are
skipped unless MLA_RUN_UNVALIDATED=1 asks for its first GPU run.  (Named to run
after every validated suite.)"""
import math
import os

import numpy as np
import pytest

from workloads import make_case, workload

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(os.environ.get("MLA_RUN_UNVALIDATED") != "1",
                       reason="candidate kernel not yet run on a GPU: set MLA_RUN_UNVALIDATED=1 "
                              "for its first run"),
]

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from tests.test_gpu_parity import check, run_gpu  # noqa: E402


@pytest.fixture(autouse=True)
def w8(monkeypatch):
    monkeypatch.setenv("MLA_DECODE_KERNEL", "w8")


@pytest.mark.parametrize("kv_lens,q_lens,nwg", [
    ([1, 15, 16, 17, 129, 31, 33], [1, 1, 2, 1, 2, 1, 2], 12),
    ([3000, 700, 65, 1800], [1, 2, 1, 2], 1),
    ([3000, 700, 65, 1800], [1, 2, 1, 2], 256),
    ([0, 200, 64], [0, 2, 1], 5),
])
def test_w8_small_cases(kv_lens, q_lens, nwg):
    case = make_case(kv_lens=kv_lens, q_lens=q_lens, seed=37, max_q_len=2,
                     sm_scale=1 / math.sqrt(192))
    print(f"w8: lengths {kv_lens} q {q_lens} workgroups {nwg}", flush=True)
    (out, lse), _ = run_gpu(case, num_workgroups=nwg)
    check(case, out, lse)


def test_w8_restarts():
    case = make_case(kv_lens=[2000, 513], q_lens=[1, 2], seed=18, q_std=8.0,
                     sm_scale=1 / math.sqrt(192))
    print("w8: peaky softmax", flush=True)
    (out, lse), _ = run_gpu(case)
    check(case, out, lse)


def test_w8_deepseek_v3_decode():
    case = workload("v3_decode_bf16")
    print("w8: v3_decode_bf16", flush=True)
    (out, lse), _ = run_gpu(case)
    check(case, out, lse)


@pytest.mark.parametrize("kv_lens,q_lens,nwg,P", [
    ([1, 15, 16, 17, 31, 33, 63, 65, 129], [1, 1, 2, 1, 2, 1, 2, 1, 2], 12, 64),
    ([3000, 700, 65, 1800], [1, 2, 1, 2], 1, 64),
    ([3000, 700, 65, 1800], [1, 2, 1, 2], 256, 256),
    ([0, 200, 64], [0, 2, 1], 5, 64),
])
def test_w8_e4m3_small_cases(kv_lens, q_lens, nwg, P):
    case = make_case(kv_lens=kv_lens, q_lens=q_lens, seed=39, max_q_len=2, page_size=P,
                     kv_dtype="fp8_e4m3", sm_scale=1 / math.sqrt(192))
    print(f"w8 e4m3: lengths {kv_lens} q {q_lens} workgroups {nwg} pages {P}", flush=True)
    (out, lse), pl = run_gpu(case, num_workgroups=nwg, phases=1)
    assert pl.phases == 1
    check(case, out, lse)


def test_w8_e4m3_long_context():
    case = workload("long_ctx_fp8")
    print("w8: long_ctx_fp8 (every sequence)", flush=True)
    (out, lse), pl = run_gpu(case, phases=1)
    assert pl.phases == 1
    check(case, out, lse)

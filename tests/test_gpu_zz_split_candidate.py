"""GPU parity of the candidate decode kernel whose pairs of waves share 32
rows (decode_split_kernel.hip, selected by MLA_DECODE_KERNEL=split for
one-phase plans, bf16 or e4m3 cache) against the float64 oracle, at the
decode bars.

The candidate has passed the CPU emulator (both copy-landing modes, the
lockstep and drift schedules, planted synchronisation mistakes;
tests/test_kernel_emulated.py) and the machine-code checks
(tests/test_kernel_isa.py) but has not run on a GPU yet, so these cases are
skipped unless MLA_RUN_UNVALIDATED=1 asks for its first GPU run.  (Named to
run after every validated suite.)"""
import math
import os

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
def split(monkeypatch):
    monkeypatch.setenv("MLA_DECODE_KERNEL", "split")


@pytest.mark.parametrize("kv_lens,q_lens,nwg,P", [
    ([1, 15, 16, 17, 129, 31, 33], [1, 1, 2, 1, 2, 1, 2], 12, 64),
    ([3000, 700, 65, 1800], [1, 2, 1, 2], 1, 16),
    ([3000, 700, 65, 1800], [1, 2, 1, 2], 256, 256),
    ([0, 200, 64], [0, 2, 1], 5, 64),
])
def test_split_small_cases(kv_lens, q_lens, nwg, P):
    case = make_case(kv_lens=kv_lens, q_lens=q_lens, seed=37, max_q_len=2, page_size=P,
                     sm_scale=1 / math.sqrt(192))
    print(f"split: lengths {kv_lens} q {q_lens} workgroups {nwg} pages {P}", flush=True)
    (out, lse), pl = run_gpu(case, num_workgroups=nwg, phases=1)
    assert pl.phases == 1
    check(case, out, lse)


def test_split_peaky_softmax():
    case = make_case(kv_lens=[2000, 513], q_lens=[1, 2], seed=18, q_std=8.0,
                     sm_scale=1 / math.sqrt(192))
    print("split: peaky softmax", flush=True)
    (out, lse), _ = run_gpu(case, phases=1)
    check(case, out, lse)


@pytest.mark.parametrize("kv_lens,q_lens,nwg,P", [
    ([1, 15, 16, 17, 31, 33, 63, 65, 129], [1, 1, 2, 1, 2, 1, 2, 1, 2], 12, 64),
    ([3000, 700, 65, 1800], [1, 2, 1, 2], 1, 64),
    ([3000, 700, 65, 1800], [1, 2, 1, 2], 256, 256),
    ([0, 200, 64], [0, 2, 1], 5, 64),
])
def test_split_e4m3_small_cases(kv_lens, q_lens, nwg, P):
    case = make_case(kv_lens=kv_lens, q_lens=q_lens, seed=39, max_q_len=2, page_size=P,
                     kv_dtype="fp8_e4m3", sm_scale=1 / math.sqrt(192))
    print(f"split e4m3: lengths {kv_lens} q {q_lens} workgroups {nwg} pages {P}", flush=True)
    (out, lse), pl = run_gpu(case, num_workgroups=nwg, phases=1)
    assert pl.phases == 1
    check(case, out, lse)


@pytest.mark.parametrize("name", ["v3_decode_bf16", "mtp_verify_bf16", "long_ctx_fp8",
                                  "ragged_serving_bf16"])
def test_split_full_size_workloads(name):
    # every sequence of the four workloads at full size, in the launch
    # configuration bench.py times, one-phase plans
    case = workload(name)
    print(f"split: {name}", flush=True)
    (out, lse), pl = run_gpu(case, phases=1)
    assert pl.phases == 1
    worst, rel = check(case, out, lse)
    print(f"split: {name}: max-abs {worst:.3g} rel-L2 {rel:.3g}", flush=True)


def test_split_graph_replay_with_new_lengths():
    # fwd + combine captured once in a HIP graph over a fixed-shape plan and
    # replayed for other lengths (the library's graph test, with the
    # candidate selected): each replay equal, bit for bit, to the eager call
    from tests import test_gpu_graph
    print("split: graph replay", flush=True)
    test_gpu_graph.test_graph_replay_with_new_lengths()


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8_e4m3"])
def test_split_page_relayout_is_bitwise_identical(kv_dtype):
    # the library's relayout check with the candidate selected: pages moved
    # in the pool, the same plan, the same bits
    from tests import test_gpu_parity
    print(f"split: page relayout {kv_dtype}", flush=True)
    test_gpu_parity.test_page_relayout_is_bitwise_identical(kv_dtype, 1)


def test_split_repeat_runs_bitwise_equal():
    # 20 runs of one plan, bit for bit equal (a race canary)
    from tests import test_gpu_parity
    print("split: repeat runs", flush=True)
    test_gpu_parity.test_repeat_runs_bitwise_equal(1)


def test_split_unused_block_table_entries_never_read():
    from tests import test_gpu_parity
    print("split: unused block-table entries", flush=True)
    test_gpu_parity.test_unused_block_table_entries_never_read()

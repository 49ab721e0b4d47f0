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


def test_w8_peaky_softmax():
    case = make_case(kv_lens=[2000, 513], q_lens=[1, 2], seed=18, q_std=8.0,
                     sm_scale=1 / math.sqrt(192))
    print("w8: peaky softmax", flush=True)
    (out, lse), _ = run_gpu(case)
    check(case, out, lse)


@pytest.mark.parametrize("name", ["v3_decode_bf16", "mtp_verify_bf16", "long_ctx_fp8",
                                  "ragged_serving_bf16"])
def test_w8_full_size_workloads(name):
    # every sequence of the four workloads at full size, in the launch
    # configuration bench.py times, one-phase plans
    case = workload(name)
    print(f"w8: {name}", flush=True)
    (out, lse), pl = run_gpu(case, phases=1)
    assert pl.phases == 1
    worst, rel = check(case, out, lse)
    print(f"w8: {name}: max-abs {worst:.3g} rel-L2 {rel:.3g}", flush=True)


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


def test_w8_combine_of_bf16_partials_matches_combine_ref():
    # the merge the candidate's split rows take: bf16 partials (the first half
    # of the fp32 partial area), fp32 LSE where it always is
    import oracle
    import mla_paged_decode_absorbed_amd as mla
    from tests.test_gpu_parity import DEV, as_f64, shape_of
    case = make_case(kv_lens=[3000, 2500], q_lens=[2, 1], seed=25, sm_scale=1 / math.sqrt(192))
    shape = shape_of(case)
    pl = mla.plan(shape, case.kv_lens, case.q_lens, num_workgroups=64)
    assert pl.info.num_combine > 0 and pl.phases == 1
    rng = np.random.default_rng(0)
    P = pl.info.num_partials
    po = torch.from_numpy(rng.standard_normal((P, 128, 512)).astype(np.float32))
    po_b = po.to(torch.bfloat16)
    plse = (rng.standard_normal((P, 128)) * 3).astype(np.float32)
    plse[::5, ::7] = -np.inf      # empty partials: their O (NaN here) must be ignored
    po_b[::5, ::7] = float("nan")
    print("w8: combine of bf16 partials", flush=True)
    ws = mla.alloc_workspace(pl)
    ws.view(torch.bfloat16)[: P * 128 * 512].copy_(po_b.reshape(-1))
    base = ws.view(torch.float32)
    base[P * 128 * 512: P * 128 * 512 + P * 128].copy_(torch.from_numpy(plse.reshape(-1)))
    out = torch.zeros((case.batch, 2, case.num_heads, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.zeros((case.batch, 2, case.num_heads), dtype=torch.float32, device=DEV)
    mla.combine(shape, pl, ws, torch.from_numpy(case.q_lens).to(DEV), out, lse)
    torch.cuda.synchronize()
    o, l = as_f64(out, lse)
    pof = po_b.float().numpy().astype(np.float64)
    for b, row0, first, n in pl.combine_entries():
        Oc, Lc = oracle.combine_ref(pof[first:first + n], plse[first:first + n])
        rows = min(128, int(case.q_lens[b]) * case.num_heads - int(row0))
        for r in range(rows):
            t, h = divmod(int(row0) + r, case.num_heads)
            if np.isneginf(Lc[r]):
                assert np.isneginf(l[b, t, h]) and np.all(o[b, t, h] == 0)
                continue
            assert abs(l[b, t, h] - Lc[r]) <= 1e-4 * max(1.0, abs(Lc[r]))
            assert np.abs(o[b, t, h] - Oc[r]).max() <= 4e-3 * np.abs(Oc[r]).max()


def test_w8_graph_replay_with_new_lengths():
    # fwd + combine captured once in a HIP graph over a fixed-shape plan and
    # replayed for other lengths (the library's graph test, with the
    # candidate selected): each replay equal, bit for bit, to the eager call
    from tests import test_gpu_graph
    print("w8: graph replay", flush=True)
    test_gpu_graph.test_graph_replay_with_new_lengths()


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8_e4m3"])
def test_w8_page_relayout_is_bitwise_identical(kv_dtype):
    # the library's relayout check with the candidate selected: pages moved
    # in the pool, the same plan, the same bits
    from tests import test_gpu_parity
    print(f"w8: page relayout {kv_dtype}", flush=True)
    test_gpu_parity.test_page_relayout_is_bitwise_identical(kv_dtype, 1)


def test_w8_repeat_runs_bitwise_equal():
    # 20 runs of one plan, bit for bit equal (a race canary)
    from tests import test_gpu_parity
    print("w8: repeat runs", flush=True)
    test_gpu_parity.test_repeat_runs_bitwise_equal(1)


def test_w8_unused_block_table_entries_never_read():
    from tests import test_gpu_parity
    print("w8: unused block-table entries", flush=True)
    test_gpu_parity.test_unused_block_table_entries_never_read()

"""Plans for a fixed launch shape (``mla_decode_plan_fixed``) on the GPU:
eager parity, and a HIP graph of mla_decode_fwd + mla_combine captured once
and replayed for new lengths, each replay checked against the oracle and,
bit for bit, against the eager call with the same plan.
"""
import math

import numpy as np
import pytest

from workloads import make_case

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import mla_paged_decode_absorbed_amd as mla  # noqa: E402
from tests.test_gpu_parity import SENTINEL, check, run_gpu, shape_of  # noqa: E402

DEV = "cuda"


@pytest.mark.parametrize("kv_lens,q_lens,nwg,dtype", [
    ([700, 130, 5, 2000], [2, 2, 1, 1], 256, "bf16"),
    ([3000, 64, 1], [1, 1, 1], 96, "bf16"),
    ([900, 4000], [1, 2], 256, "fp8_e4m3"),
])
def test_fixed_shape_plan_parity(kv_lens, q_lens, nwg, dtype):
    case = make_case(kv_lens=kv_lens, q_lens=q_lens, seed=47, kv_dtype=dtype,
                     sm_scale=1 / math.sqrt(192), max_q_len=2)
    shape = shape_of(case)
    pl = mla.plan(shape, case.kv_lens, case.q_lens, num_workgroups=nwg, fixed=True)
    assert pl.info.num_workgroups == nwg
    (out, lse), _ = run_gpu(case, pl=pl)
    check(case, out, lse)


B, QMAX, H, P = 8, 2, 128, 64
LENGTH_SETS = [
    ([3000, 17, 640, 2, 1200, 90, 4096, 300], [2, 1, 2, 2, 1, 0, 1, 2]),
    ([64, 2500, 2500, 2500, 3, 700, 1, 129], [1, 2, 2, 1, 2, 2, 1, 1]),
    ([4096, 4096, 4096, 4096, 4096, 4096, 4096, 4096], [2] * 8),
]


def _cases():
    return [make_case(kv_lens=kv, q_lens=ql, seed=60 + i, sm_scale=1 / math.sqrt(192),
                      max_q_len=QMAX) for i, (kv, ql) in enumerate(LENGTH_SETS)]


def test_graph_replay_with_new_lengths():
    cases = _cases()
    pool = max(c.num_pages for c in cases)
    maxp = max(c.max_pages for c in cases)
    shape = mla.Shape.make(batch=B, num_heads=H, max_q_len=QMAX, page_size=P, num_pages=pool,
                           max_pages_per_seq=maxp, causal=True)
    plans = [mla.plan(shape, c.kv_lens, c.q_lens, fixed=True, upload=False) for c in cases]
    info = plans[0].info
    for p in plans[1:]:   # one set of launch bounds serves every lengths of the shape
        for f in ("num_workgroups", "num_partials", "num_combine", "phases", "plan_bytes",
                  "workspace_bytes"):
            assert getattr(p.info, f) == getattr(info, f), f

    q_d = torch.empty((B, QMAX, H, 576), dtype=torch.bfloat16, device=DEV)
    kv_d = torch.empty((pool, P, 576), dtype=torch.bfloat16, device=DEV)
    bt_d = torch.empty((B, maxp), dtype=torch.int32, device=DEV)
    kvl_d = torch.empty(B, dtype=torch.int32, device=DEV)
    ql_d = torch.empty(B, dtype=torch.int32, device=DEV)
    plan_d = torch.empty(info.plan_bytes // 4, dtype=torch.int32, device=DEV)
    ws_d = torch.empty(info.workspace_bytes, dtype=torch.uint8, device=DEV)
    out_d = torch.empty((B, QMAX, H, 512), dtype=torch.bfloat16, device=DEV)
    lse_d = torch.empty((B, QMAX, H), dtype=torch.float32, device=DEV)

    def load(i):
        c = cases[i]
        q_d.copy_(torch.from_numpy(c.q.view(np.int16)).view(torch.bfloat16))
        kv = np.full((pool, P, 576), 0x7FC0, np.uint16)      # unused pages: NaN
        kv[:c.num_pages] = c.kv
        kv_d.copy_(torch.from_numpy(kv.view(np.int16)).view(torch.bfloat16))
        bt = np.full((B, maxp), -1, np.int32)
        bt[:, :c.max_pages] = c.block_table
        bt_d.copy_(torch.from_numpy(bt))
        kvl_d.copy_(torch.from_numpy(c.kv_lens))
        ql_d.copy_(torch.from_numpy(c.q_lens))
        plan_d.copy_(torch.from_numpy(plans[i].host))
        out_d.view(torch.int16).fill_(SENTINEL)
        lse_d.fill_(12345.0)
        torch.cuda.synchronize()

    pl_dev = mla.Plan(info=info, host=plans[0].host, device=plan_d)

    def step():
        mla.decode_fwd(shape, pl_dev, q_d, kv_d, bt_d, kvl_d, ql_d, cases[0].sm_scale, out_d,
                       lse_d, ws_d)
        mla.combine(shape, pl_dev, ws_d, ql_d, out_d, lse_d)

    # eager reference of every lengths set with the same buffers and plan layout
    eager = []
    for i in range(len(cases)):
        load(i)
        step()
        torch.cuda.synchronize()
        check(cases[i], out_d, lse_d)
        eager.append((out_d.clone(), lse_d.clone()))

    load(0)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    for rep, i in enumerate([0, 1, 2, 1, 0, 2]):
        load(i)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_d.view(torch.int16), eager[i][0].view(torch.int16)), rep
        assert torch.equal(lse_d, eager[i][1]), rep
        check(cases[i], out_d, lse_d)
        # the program's own eager work between replays
        other = make_case(kv_lens=[300, 65], q_lens=[1, 2], seed=90 + rep,
                          sm_scale=1 / math.sqrt(192))
        (o2, l2), _ = run_gpu(other, num_workgroups=32)
        check(other, o2, l2)

"""Plans for a fixed launch shape on the GPU: the host planner's
(``mla_decode_plan_fixed``) and the device planner's
(``mla_decode_plan_device``, which must equal it word for word).  Eager
parity, and HIP graphs captured once and replayed for new lengths (fwd +
combine after a host plan upload; planner + fwd + combine reading the lengths
on the GPU), each replay checked against the oracle and, bit for bit, against
the eager call.
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


# ---------------------------------------------------------------- device-side planner

def _device_lengths(c):
    return torch.from_numpy(c.kv_lens).to(DEV), torch.from_numpy(c.q_lens).to(DEV)


@pytest.mark.parametrize("phases", [1, 4])
def test_device_plan_equals_host_plan(monkeypatch, phases):
    monkeypatch.setenv("MLA_PHASES", str(phases) if phases > 1 else "")
    cases = _cases()
    pool = max(c.num_pages for c in cases)
    maxp = max(c.max_pages for c in cases)
    shape = mla.Shape.make(batch=B, num_heads=H, max_q_len=QMAX, page_size=P, num_pages=pool,
                           max_pages_per_seq=maxp, causal=True)
    status = torch.full((1,), -1, dtype=torch.int32, device=DEV)
    for c in cases:
        host = mla.plan(shape, c.kv_lens, c.q_lens, fixed=True, upload=False)
        kvl, ql = _device_lengths(c)
        dp = mla.plan_device(shape, kvl, ql, status=status)
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        n = int(host.host[10]) + 4 * int(host.host[4])
        assert np.array_equal(dp.device[:n].cpu().numpy(), host.host[:n])
        for f in ("num_workgroups", "num_items", "num_partials", "num_combine", "phases",
                  "plan_bytes", "workspace_bytes"):
            assert getattr(dp.info, f) == getattr(host.info, f), f


def test_device_plan_rejects_bad_lengths_and_decode_writes_nothing():
    c = make_case(kv_lens=[300, 65], q_lens=[1, 2], seed=71, sm_scale=1 / math.sqrt(192),
                  max_q_len=2)
    shape = shape_of(c)
    kvl = torch.tensor([300, 1], dtype=torch.int32, device=DEV)   # causal: 1 key < 2 tokens
    ql = torch.from_numpy(c.q_lens).to(DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    dp = mla.plan_device(shape, kvl, ql, status=status)
    q = torch.from_numpy(c.q.view(np.int16)).view(torch.bfloat16).to(DEV)
    kv = torch.from_numpy(c.kv.view(np.int16)).view(torch.bfloat16).to(DEV)
    bt = torch.from_numpy(c.block_table).to(DEV)
    out = torch.full((c.batch, c.max_q_len, c.num_heads, 512), SENTINEL, dtype=torch.int16,
                     device=DEV)
    lse = torch.full((c.batch, c.max_q_len, c.num_heads), 12345.0, dtype=torch.float32,
                     device=DEV)
    mla.decode(shape, dp, q, kv, bt, kvl, ql, c.sm_scale, out=out.view(torch.bfloat16), lse=lse)
    torch.cuda.synchronize()
    assert int(status.item()) == 2                     # MLA_ERR_BAD_SHAPE
    assert bool((out == SENTINEL).all()) and bool((lse == 12345.0).all())


def test_graph_of_plan_decode_combine_with_device_lengths():
    # the whole step in one graph: the planner reads the lengths on the GPU
    cases = _cases()
    pool = max(c.num_pages for c in cases)
    maxp = max(c.max_pages for c in cases)
    shape = mla.Shape.make(batch=B, num_heads=H, max_q_len=QMAX, page_size=P, num_pages=pool,
                           max_pages_per_seq=maxp, causal=True)
    q_d = torch.empty((B, QMAX, H, 576), dtype=torch.bfloat16, device=DEV)
    kv_d = torch.empty((pool, P, 576), dtype=torch.bfloat16, device=DEV)
    bt_d = torch.empty((B, maxp), dtype=torch.int32, device=DEV)
    kvl_d = torch.empty(B, dtype=torch.int32, device=DEV)
    ql_d = torch.empty(B, dtype=torch.int32, device=DEV)
    out_d = torch.empty((B, QMAX, H, 512), dtype=torch.bfloat16, device=DEV)
    lse_d = torch.empty((B, QMAX, H), dtype=torch.float32, device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)

    def load(i):
        c = cases[i]
        q_d.copy_(torch.from_numpy(c.q.view(np.int16)).view(torch.bfloat16))
        kv = np.full((pool, P, 576), 0x7FC0, np.uint16)
        kv[:c.num_pages] = c.kv
        kv_d.copy_(torch.from_numpy(kv.view(np.int16)).view(torch.bfloat16))
        bt = np.full((B, maxp), -1, np.int32)
        bt[:, :c.max_pages] = c.block_table
        bt_d.copy_(torch.from_numpy(bt))
        kvl_d.copy_(torch.from_numpy(c.kv_lens))
        ql_d.copy_(torch.from_numpy(c.q_lens))
        out_d.view(torch.int16).fill_(SENTINEL)
        lse_d.fill_(12345.0)
        status.fill_(-1)
        torch.cuda.synchronize()

    load(0)
    dp = mla.plan_device(shape, kvl_d, ql_d, status=status)     # allocates the plan buffer
    ws_d = torch.empty(dp.info.workspace_bytes, dtype=torch.uint8, device=DEV)

    def step():
        mla.plan_device(shape, kvl_d, ql_d, plan_buf=dp.device, status=status,
                        num_workgroups=dp.info.num_workgroups)
        mla.decode_fwd(shape, dp, q_d, kv_d, bt_d, kvl_d, ql_d, cases[0].sm_scale, out_d, lse_d,
                       ws_d)
        mla.combine(shape, dp, ws_d, ql_d, out_d, lse_d)

    eager = []
    for i in range(len(cases)):
        load(i)
        step()
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        check(cases[i], out_d, lse_d)
        eager.append((out_d.clone(), lse_d.clone()))

    load(0)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep, i in enumerate([1, 0, 2, 2, 1]):
        load(i)
        g.replay()
        torch.cuda.synchronize()
        assert int(status.item()) == 0, rep
        assert torch.equal(out_d.view(torch.int16), eager[i][0].view(torch.int16)), rep
        assert torch.equal(lse_d, eager[i][1]), rep
        check(cases[i], out_d, lse_d)
        other = make_case(kv_lens=[500, 33], q_lens=[2, 1], seed=95 + rep,
                          sm_scale=1 / math.sqrt(192))
        (o2, l2), _ = run_gpu(other, num_workgroups=24)
        check(other, o2, l2)

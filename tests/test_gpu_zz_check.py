"""The debug validation kernel (mla_decode_check) on MI355X, and the checked
mode of the binding (MLA_DEBUG_CHECK=1): valid inputs pass and the decode
runs; a stale plan or a page id outside the pool is reported and the decode
is not launched.  The same cases run on the CPU emulator in
tests/test_check_emulated.py.  (Named to run after the decode suites.)"""
import math

import numpy as np
import pytest

from workloads import make_case

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import mla_paged_decode_absorbed_amd as mla  # noqa: E402

DEV = "cuda"


def _setup(case, plan_lens=None, nwg=16):
    shape = mla.Shape.make(batch=case.batch, num_heads=case.num_heads, max_q_len=case.max_q_len,
                           page_size=case.page_size, num_pages=case.num_pages,
                           max_pages_per_seq=case.max_pages, causal=case.causal)
    pl = mla.plan(shape, case.kv_lens if plan_lens is None else plan_lens, case.q_lens,
                  num_workgroups=nwg, device=DEV)
    bt = torch.from_numpy(case.block_table).to(DEV)
    kvl = torch.from_numpy(case.kv_lens).to(DEV)
    ql = torch.from_numpy(case.q_lens).to(DEV)
    return shape, pl, bt, kvl, ql


def _case():
    return make_case(kv_lens=[700, 64, 1234, 5], q_lens=[2, 1, 1, 2], seed=3, max_q_len=2,
                     sm_scale=1 / math.sqrt(192))


def test_valid_inputs_pass():
    case = _case()
    shape, pl, bt, kvl, ql = _setup(case)
    print("check: valid inputs", flush=True)
    assert mla.check(shape, pl, bt, kvl, ql) == (0, 0)


def test_stale_plan_and_bad_page_are_reported():
    case = _case()
    longer = case.kv_lens.copy()
    longer[2] += 100
    shape, pl, bt, kvl, ql = _setup(case, plan_lens=longer)
    print("check: stale plan", flush=True)
    assert mla.check(shape, pl, bt, kvl, ql)[0] == 4
    shape, pl, bt, kvl, ql = _setup(case)
    bt2 = bt.clone()
    bt2[2, 5] = case.num_pages
    print("check: page outside the pool", flush=True)
    assert mla.check(shape, pl, bt2, kvl, ql) == (3, 2)


def test_checked_decode_raises_before_launch(monkeypatch):
    case = _case()
    longer = case.kv_lens.copy()
    longer[2] += 100
    shape, pl, bt, kvl, ql = _setup(case, plan_lens=longer)
    q = torch.from_numpy(case.q.view(np.int16)).view(torch.bfloat16).to(DEV)
    kv = torch.from_numpy(case.kv.view(np.int16)).view(torch.bfloat16).to(DEV)
    monkeypatch.setenv("MLA_DEBUG_CHECK", "1")
    print("check: checked decode with a stale plan", flush=True)
    with pytest.raises(mla.MLAInputError) as e:
        mla.decode(shape, pl, q, kv, bt, kvl, ql, case.sm_scale)
    assert e.value.code == 4
    # with the plan for these lengths the checked decode runs
    shape, pl, bt, kvl, ql = _setup(case)
    out, lse = mla.decode(shape, pl, q, kv, bt, kvl, ql, case.sm_scale)
    torch.cuda.synchronize()
    assert torch.isfinite(out[2, :1].float()).all()

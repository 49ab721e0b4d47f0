"""GPU parity of the cache append (``mla_kv_append`` through the C ABI) with
the oracle: bit-exact over the whole cache, every scale and the skip count;
then the decode of an appended cache against the decode oracle.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import append_ref
from tests.append_cases import make_append_case
from workloads import make_case, workload

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import mla_paged_decode_absorbed_amd as mla  # noqa: E402

DEV = "cuda"


def test_hardware_e4m3_conversion_matches_definition():
    # v_cvt_pk_fp8_f32, which the kernel rounds with, against a plain encoder
    # of the e4m3 definition for every fp32 value in [-448, 448]
    import ctypes
    import os
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "gpu_checks",
                        "libe4m3_convert_check.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: run __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    lib.e4m3_convert_check.restype = ctypes.c_int
    lib.e4m3_convert_check.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    bad = torch.zeros(1, dtype=torch.int64, device=DEV)
    first = torch.full((16,), -1, dtype=torch.int32, device=DEV)
    stream = torch.cuda.current_stream()
    assert lib.e4m3_convert_check(bad.data_ptr(), first.data_ptr(), stream.cuda_stream) == 0
    torch.cuda.synchronize()
    assert int(bad.item()) == 0, [hex(v & 0xFFFFFFFF) for v in first.cpu().tolist()]


def _shape(c, batch=None):
    return mla.Shape.make(batch=batch if batch is not None else len(c["kv_lens"]), num_heads=1,
                          max_q_len=1, page_size=c["page_size"], num_pages=c["kv"].shape[0],
                          max_pages_per_seq=c["block_table"].shape[1],
                          kv_dtype=mla.KV_BF16 if c["kv_dtype"] == "bf16" else mla.KV_FP8_E4M3)


def _gpu_append(c, use_new_lens=True, with_counter=True):
    kv = torch.from_numpy(c["kv"].view(np.int16) if c["kv_dtype"] == "bf16" else c["kv"]).to(DEV)
    sc = None if c["kv_scale"] is None else torch.from_numpy(c["kv_scale"]).to(DEV)
    rows = torch.from_numpy(c["new_rows_bits"].view(np.int16)).view(torch.bfloat16).to(DEV)
    bt = torch.from_numpy(c["block_table"]).to(DEV)
    kvl = torch.from_numpy(c["kv_lens"]).to(DEV)
    nl = torch.from_numpy(c["new_lens"]).to(DEV) if use_new_lens else None
    sk = torch.zeros(1, dtype=torch.int32, device=DEV) if with_counter else None
    mla.kv_append(_shape(c), rows, bt, kvl, kv, new_lens=nl, kv_scale=sc, skipped=sk)
    torch.cuda.synchronize()
    out = kv.cpu().numpy()
    out = out.view(np.uint16) if c["kv_dtype"] == "bf16" else out
    return (out, None if sc is None else sc.cpu().numpy(),
            None if sk is None else int(sk.cpu().item()))


def _check(c, use_new_lens=True, with_counter=True):
    nl = c["new_lens"] if use_new_lens else None
    want_kv, want_sc, want_sk = append_ref.kv_append_ref(
        c["kv"], c["kv_scale"], c["block_table"], c["kv_lens"], nl, c["new_rows_bits"],
        c["page_size"], c["kv_dtype"])
    got_kv, got_sc, got_sk = _gpu_append(c, use_new_lens, with_counter)
    assert np.array_equal(got_kv, want_kv)
    if c["kv_dtype"] == "fp8_e4m3":
        assert np.array_equal(got_sc.view(np.uint32), want_sc.view(np.uint32))
    if with_counter:
        assert got_sk == want_sk
    return want_sk


@pytest.mark.parametrize("kv_dtype,P", [("bf16", 16), ("bf16", 64), ("fp8_e4m3", 64),
                                        ("fp8_e4m3", 256)])
def test_decode_step_append(kv_dtype, P):
    c = make_append_case([70, 5, 129, 64, 3, 1, 200], [2, 5, 1, 0, 3, 1, 8], P, kv_dtype, seed=3)
    assert _check(c) == 0


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8_e4m3"])
def test_rows_outside_the_pool_are_skipped(kv_dtype):
    c = make_append_case([70, 5, 129, 64, 3], [2, 5, 1, 2, 3], 64, kv_dtype, seed=4)
    bt = c["block_table"]
    bt[0, 69 // 64] = -1
    bt[2, 128 // 64] = c["kv"].shape[0]
    c["kv_lens"][4] = 1
    c["new_lens"][3] = 9
    assert _check(c) == 2 + 1 + 2 + c["new_rows_bits"].shape[1]


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8_e4m3"])
def test_without_lengths_or_counter(kv_dtype):
    c = make_append_case([70, 130, 64], [4, 4, 4], 64, kv_dtype, seed=5)
    _check(c, use_new_lens=False, with_counter=False)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8_e4m3"])
def test_prompt_sized_append(kv_dtype):
    c = make_append_case([9000, 7000, 12000], [9000, 4000, 11000], 64, kv_dtype, seed=6,
                         max_new=11000)
    assert _check(c) == 0


def test_empty_batch_is_a_noop():
    c = make_append_case([70], [2], 64, "bf16", seed=8)
    kv = torch.from_numpy(c["kv"].view(np.int16)).to(DEV)
    before = kv.clone()
    rows = torch.zeros((0, 2, 576), dtype=torch.bfloat16, device=DEV)
    empty = torch.zeros(0, dtype=torch.int32, device=DEV)
    bt = torch.zeros((0, c["block_table"].shape[1]), dtype=torch.int32, device=DEV)
    mla.kv_append(_shape(c, batch=0), rows, bt, empty, kv, new_lens=empty)
    torch.cuda.synchronize()
    assert torch.equal(kv, before)


def _wipe_and_rows(case):
    """NaN the q_b newest rows of every sequence and return them as new rows."""
    P, qmax = case.page_size, case.max_q_len
    rows = np.zeros((case.batch, qmax, 576), np.uint16)
    kv = case.kv.copy()
    for b in range(case.batch):
        L, n = int(case.kv_lens[b]), int(case.q_lens[b])
        for t in range(n):
            p = L - n + t
            page, slot = case.block_table[b, p // P], p % P
            rows[b, t] = case.kv[page, slot]
            kv[page, slot] = 0x7FC0
    return kv, rows


def _decode_gpu(case, kv_np, kv_scale_np):
    shape = mla.Shape.make(batch=case.batch, num_heads=case.num_heads, max_q_len=case.max_q_len,
                           page_size=case.page_size, num_pages=case.num_pages,
                           max_pages_per_seq=case.max_pages,
                           kv_dtype=mla.KV_BF16 if case.kv_dtype == "bf16" else mla.KV_FP8_E4M3,
                           causal=case.causal)
    q = torch.from_numpy(case.q.view(np.int16)).view(torch.bfloat16).to(DEV)
    if case.kv_dtype == "bf16":
        kv = torch.from_numpy(kv_np.view(np.int16)).view(torch.bfloat16).to(DEV)
    else:
        kv = torch.from_numpy(kv_np).to(DEV)
    sc = None if kv_scale_np is None else torch.from_numpy(kv_scale_np).to(DEV)
    bt = torch.from_numpy(case.block_table).to(DEV)
    kvl = torch.from_numpy(case.kv_lens).to(DEV)
    ql = torch.from_numpy(case.q_lens).to(DEV)
    pl = mla.plan(shape, case.kv_lens, case.q_lens)
    return shape, q, kv, sc, bt, kvl, ql, pl


def test_append_then_decode_bf16():
    # a decode step: the q_b new tokens are appended, then attended to
    case = make_case(kv_lens=[300, 1000, 77, 64], q_lens=[2, 1, 2, 1], seed=12,
                     sm_scale=1 / math.sqrt(192), max_q_len=2)
    wiped, rows = _wipe_and_rows(case)
    shape, q, kv, sc, bt, kvl, ql, pl = _decode_gpu(case, wiped, None)
    mla.kv_append(shape, torch.from_numpy(rows.view(np.int16)).view(torch.bfloat16).to(DEV),
                  bt, kvl, kv, new_lens=ql)
    out, lse = mla.decode(shape, pl, q, kv, bt, kvl, ql, case.sm_scale)
    torch.cuda.synchronize()
    assert np.array_equal(kv.view(torch.int16).cpu().numpy().view(np.uint16), case.kv)
    O, L = oracle.mla_decode_ref(case)
    o = out.float().cpu().numpy().astype(np.float64)
    lse_np = lse.cpu().numpy()
    num = den = 0.0
    for b in range(case.batch):
        n = int(case.q_lens[b])
        assert np.abs(o[b, :n] - O[b, :n]).max() <= 2e-2
        assert np.abs(lse_np[b, :n] - L[b, :n]).max() <= 1e-3
        num += float(((o[b, :n] - O[b, :n]) ** 2).sum())
        den += float((O[b, :n] ** 2).sum())
    assert math.sqrt(num / den) <= 5e-3


def test_append_then_decode_e4m3():
    case = make_case(kv_lens=[300, 1000, 77, 640], q_lens=[2, 1, 2, 1], seed=13,
                     sm_scale=1 / math.sqrt(192), max_q_len=2, kv_dtype="fp8_e4m3")
    rng = np.random.default_rng(14)
    new_rows = torch.from_numpy(rng.standard_normal((case.batch, 2, 576)).astype(np.float32) * 0.5)
    new_bits = new_rows.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    want_kv, want_sc, _ = append_ref.kv_append_ref(case.kv, case.kv_scale, case.block_table,
                                                   case.kv_lens, case.q_lens, new_bits,
                                                   case.page_size, "fp8_e4m3")
    shape, q, kv, sc, bt, kvl, ql, pl = _decode_gpu(case, case.kv, case.kv_scale)
    mla.kv_append(shape, torch.from_numpy(new_bits.view(np.int16)).view(torch.bfloat16).to(DEV),
                  bt, kvl, kv, new_lens=ql, kv_scale=sc)
    out, lse = mla.decode(shape, pl, q, kv, bt, kvl, ql, case.sm_scale, kv_scale=sc)
    torch.cuda.synchronize()
    assert np.array_equal(kv.cpu().numpy(), want_kv)
    assert np.array_equal(sc.cpu().numpy().view(np.uint32), want_sc.view(np.uint32))
    appended = case
    appended.kv, appended.kv_scale = want_kv, want_sc
    O, L = oracle.mla_decode_ref(appended)
    o = out.float().cpu().numpy().astype(np.float64)
    num = den = 0.0
    for b in range(case.batch):
        n = int(case.q_lens[b])
        assert np.abs(o[b, :n] - O[b, :n]).max() <= 6e-2
        num += float(((o[b, :n] - O[b, :n]) ** 2).sum())
        den += float((O[b, :n] ** 2).sum())
    assert math.sqrt(num / den) <= 2e-2


def test_full_size_decode_step_append():
    # the DeepSeek-V3 decode workload's pool: one new token per sequence
    case = workload("v3_decode_bf16")
    wiped, rows = _wipe_and_rows(case)
    c = dict(kv=wiped, kv_scale=None, block_table=case.block_table, kv_lens=case.kv_lens,
             new_lens=case.q_lens.astype(np.int32), new_rows_bits=rows,
             page_size=case.page_size, kv_dtype="bf16")
    got_kv, _, sk = _gpu_append(c)
    assert sk == 0
    assert np.array_equal(got_kv, case.kv)

"""The debug validation kernel (mla_decode_check) on the CPU emulator, under
AddressSanitizer: it passes every input the planner accepts and reports each
kind of broken device-resident input (stale plan, page ids outside the pool,
bad lengths, damaged plan image) with its code and index, reading nothing
outside the buffers it is given."""
import math
import shutil

import numpy as np
import pytest

from workloads import make_case

try:
    from tests.simt_emu import harness
except ImportError:  # pragma: no cover
    harness = None

clang = shutil.which("clang++") or "/opt/rocm/llvm/bin/clang++"
pytestmark = pytest.mark.skipif(harness is None or not __import__("os").path.exists(clang),
                                reason="emulator not available")

OK, PLAN, LENGTHS, BLOCK_TABLE, ITEM, COMBINE = 0, 1, 2, 3, 4, 5


def _case(**kw):
    base = dict(kv_lens=[700, 64, 1234, 5], q_lens=[2, 1, 1, 2], seed=3,
                sm_scale=1 / math.sqrt(192), max_q_len=2)
    base.update(kw)
    return make_case(**base)


@pytest.mark.parametrize("kv_dtype,nwg,phases", [("bf16", 16, 1), ("bf16", 64, 1),
                                                 ("fp8_e4m3", 16, 1), ("bf16", 16, 4),
                                                 ("bf16", 8, 2), ("bf16", 1, 1)])
def test_planner_inputs_pass(kv_dtype, nwg, phases):
    case = _case(kv_dtype=kv_dtype)
    assert harness.run_check(case, nwg, phases=phases) == (0, OK, 0)


def test_empty_and_idle_sequences_pass():
    case = make_case(kv_lens=[0, 200, 64, 3], q_lens=[0, 2, 1, 0], seed=4, max_q_len=2,
                     sm_scale=1 / math.sqrt(192))
    assert harness.run_check(case, 12) == (0, OK, 0)


def test_stale_plan_with_shorter_device_lengths_is_an_item_error():
    case = _case()
    kvl = case.kv_lens.copy()
    kvl[2] -= 100   # the plan still reads 100 keys past sequence 2's end
    st, code, idx = harness.run_check(case, 16, plan_kv_lens=case.kv_lens, kv_lens=kvl)
    assert (st, code) == (0, ITEM)


def test_stale_plan_with_longer_device_lengths_is_caught_by_coverage():
    # every item stays inside the longer sequence, but its last keys are in no
    # item (700 -> 704 keys stays inside the sequence's 11 pages)
    case = _case()
    kvl = case.kv_lens.copy()
    kvl[0] += 4
    # the planner's own image for the new lengths passes
    assert harness.run_check(case, 16, plan_kv_lens=kvl, kv_lens=kvl) == (0, OK, 0)
    st, code, idx = harness.run_check(case, 16, plan_kv_lens=case.kv_lens, kv_lens=kvl)
    assert (st, code) == (0, ITEM)


def test_stale_plan_with_other_query_lengths():
    case = _case()
    ql = case.q_lens.copy()
    ql[0] = 1   # sequence 0's second token row block no longer exists
    st, code, idx = harness.run_check(case, 16, plan_q_lens=case.q_lens, q_lens=ql)
    assert (st, code) == (0, ITEM)


@pytest.mark.parametrize("bad", [-1, 2 ** 31 - 1, "num_pages"])
def test_block_table_entry_outside_the_pool(bad):
    case = _case()
    bt = case.block_table.copy()
    bt[2, 5] = case.num_pages if bad == "num_pages" else bad   # a page sequence 2 uses
    assert harness.run_check(case, 16, block_table=bt) == (0, BLOCK_TABLE, 2)


def test_unused_block_table_entries_are_not_checked():
    case = make_case(kv_lens=[100, 40], seed=23, extra_pages_per_seq=3,
                     sm_scale=1 / math.sqrt(192))
    bt = case.block_table.copy()
    bt[bt < 0] = np.iinfo(np.int32).max
    assert harness.run_check(case, 8, block_table=bt) == (0, OK, 0)


@pytest.mark.parametrize("which,value", [("kv", -1), ("kv", "cap"), ("q", 3), ("q", -1),
                                         ("causal", None)])
def test_bad_device_lengths(which, value):
    case = _case()
    kvl, ql = case.kv_lens.copy(), case.q_lens.copy()
    if which == "kv":
        kvl[1] = case.max_pages * case.page_size + 1 if value == "cap" else value
    elif which == "q":
        ql[1] = value
    else:
        kvl[3], ql[3] = 1, 2   # causal: fewer keys than query tokens
    st, code, idx = harness.run_check(case, 16, kv_lens=kvl, q_lens=ql)
    assert (st, code) == (0, LENGTHS)
    assert idx == (3 if which == "causal" else 1)


def _header(case, nwg):
    """(words of the plan image, the plan's items [N, 8]) for the case."""
    *_, w = harness.run_check(case, nwg, want_plan=True)
    return w, w[w[9]: w[9] + 8 * w[3]].reshape(-1, 8)


@pytest.mark.parametrize("word,value", [(0, 0), (1, 99), (2, 15), (5, 10 ** 6), (9, 10 ** 6),
                                        (11, 2)])
def test_damaged_plan_header(word, value):
    # magic, version, workgroup count, partial count, item offset, phases
    case = _case()
    assert harness.run_check(case, 16, pokes=[(word, value)]) == (0, PLAN, 0)


def test_workgroup_item_ranges_out_of_order():
    case = _case()
    w, _ = _header(case, 16)
    off = int(w[8])
    assert harness.run_check(case, 16, pokes=[(off + 3, int(w[off + 4]) + 1)])[1] == PLAN


@pytest.mark.parametrize("field,value", [(0, 4), (0, -1), (2, 32), (3, 10 ** 5), (4, 10 ** 4),
                                         (4, -2), (5, 64)])
def test_damaged_item(field, value):
    # sequence, k0 off the 64-key grid, k1 past the keys, slot, slot row
    case = _case()
    w, items = _header(case, 16)
    n = 1
    pokes = [(int(w[9]) + 8 * n + field, value)]
    st, code, idx = harness.run_check(case, 16, pokes=pokes)
    assert (st, code, idx) == (0, ITEM, n)


@pytest.mark.parametrize("field,value", [(0, 7), (2, 10 ** 4), (3, 0), (3, 10 ** 4)])
def test_damaged_combine_entry(field, value):
    case = _case()
    w, _ = _header(case, 16)
    assert int(w[4]) > 0
    pokes = [(int(w[10]) + field, value)]
    assert harness.run_check(case, 16, pokes=pokes) == (0, COMBINE, 0)


def test_lowest_code_wins():
    case = _case()
    bt = case.block_table.copy()
    bt[0, 0] = -5
    kvl = case.kv_lens.copy()
    kvl[2] = -1
    assert harness.run_check(case, 16, kv_lens=kvl, block_table=bt)[1:] == (LENGTHS, 2)


def test_every_plan_of_random_shapes_passes_and_a_damaged_one_fails():
    """Seeded random shapes, lengths (zero-length and idle sequences included),
    workgroup counts and phases: the planner's image always passes the check,
    and one damaged word in an item (its key end past the sequence) always
    fails it."""
    rng = np.random.default_rng(2024)
    for trial in range(24):
        B = int(rng.integers(1, 10))
        H = int(rng.choice([16, 32, 128]))
        qmax = int(rng.integers(1, 5))
        kvd = str(rng.choice(["bf16", "fp8_e4m3"]))
        P = int(rng.choice([64, 256] if kvd == "fp8_e4m3" else [16, 64, 256]))
        ql = rng.integers(0, qmax + 1, size=B)
        kvl = np.where(ql > 0, rng.integers(0, 3000, size=B) + ql, rng.integers(0, 50, size=B))
        phases = int(rng.choice([1, 2, 4]))
        nwg = phases * int(rng.integers(1, 24))
        case = make_case(kv_lens=kvl.tolist(), q_lens=ql.tolist(), num_heads=H, page_size=P,
                         kv_dtype=kvd, max_q_len=qmax, seed=trial, sm_scale=1 / math.sqrt(192))
        st, code, idx, w = harness.run_check(case, nwg, phases=phases, want_plan=True)
        assert (st, code, idx) == (0, OK, 0), (trial, code, idx)
        items = w[w[9]: w[9] + 8 * w[3]].reshape(-1, 8)
        if len(items):
            n = int(rng.integers(0, len(items)))
            b = int(items[n, 0])
            poke = [(int(w[9]) + 8 * n + 3, int(case.kv_lens[b]) + 1)]
            assert harness.run_check(case, nwg, phases=phases, pokes=poke)[1] == ITEM, trial

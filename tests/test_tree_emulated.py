"""Tree-shaped drafts on the CPU emulator: a non-causal decode over the prefix
(the library's decode kernels) merged with the drafts by mla_tree_attend,
against the tree oracle at the decode's tolerances, under AddressSanitizer."""
import math

import numpy as np
import pytest

from oracle import tree_ref
from tests.test_kernel_emulated import _available
from tests.tree_cases import tree_masks
from workloads import make_case

try:
    from tests.simt_emu import harness
except ImportError:  # pragma: no cover
    harness = None

pytestmark = pytest.mark.skipif(harness is None or not _available(),
                                reason="host clang++ not available")

TOL = {"bf16": (2e-2, 5e-3), "fp8_e4m3": (6e-2, 2e-2)}


def check_tree(case, mask, out_bits, lse):
    O, L = tree_ref.mla_decode_tree_ref(case, mask)
    o = harness.bf16_bits_to_f64(out_bits)
    mabs, mrel = TOL[case.kv_dtype]
    num = den = worst = 0.0
    for b in range(case.batch):
        q = int(case.q_lens[b])
        if q == 0:
            assert np.all(out_bits[b] == 0xC1C1)
            continue
        d = o[b, :q] - O[b, :q]
        assert np.all(np.isfinite(o[b, :q]))
        worst = max(worst, float(np.abs(d).max()))
        num += float((d ** 2).sum())
        den += float((O[b, :q] ** 2).sum())
        # a row with no visible key at all: O = 0 and LSE = -inf on both sides
        same_inf = np.isinf(L[b, :q]) & (lse[b, :q] == L[b, :q])
        gap = np.abs(np.where(same_inf, 0.0, lse[b, :q]) - np.where(same_inf, 0.0, L[b, :q]))
        assert float(gap.max()) <= 1e-3
        if q < case.max_q_len:
            assert np.all(out_bits[b, q:] == 0xC1C1)
    assert worst <= mabs, worst
    assert math.sqrt(num / max(den, 1e-300)) <= mrel


@pytest.mark.parametrize("kind", ["causal", "diag", "branch", "random", "none"])
def test_tree_masks_bf16(kind):
    case = make_case(kv_lens=[300, 8, 70, 4, 1000], q_lens=[4, 8, 3, 4, 0], seed=51,
                     num_heads=16, page_size=16, sm_scale=1 / math.sqrt(192), max_q_len=8)
    mask = tree_masks(case.q_lens, case.max_q_len, kind, seed=2)
    out, lse, _ = harness.run(case, 6, 1, tree_mask=mask)
    check_tree(case, mask, out, lse)


def test_tree_full_heads_and_e4m3():
    for dtype in ("bf16", "fp8_e4m3"):
        case = make_case(kv_lens=[200, 4], q_lens=[4, 4], seed=53, kv_dtype=dtype,
                         sm_scale=1 / math.sqrt(192), max_q_len=4)
        mask = tree_masks(case.q_lens, case.max_q_len, "branch", seed=3)
        out, lse, _ = harness.run(case, 8, 1, tree_mask=mask)
        check_tree(case, mask, out, lse)


@pytest.mark.parametrize("H,qmax", [(20, 4), (8, 3)])
def test_tree_partial_head_groups(H, qmax):
    # 20 heads: a second head group with one busy wave (24 workgroups, dealt
    # to XCDs); 8 heads, 3 tokens: a grid of 9, taken in plain order
    case = make_case(kv_lens=[90, 3, 400], q_lens=[qmax, 3, 2], seed=54, num_heads=H,
                     page_size=16, sm_scale=1 / math.sqrt(192), max_q_len=qmax)
    mask = tree_masks(case.q_lens, case.max_q_len, "random", seed=6)
    out, lse, _ = harness.run(case, 5, 1, tree_mask=mask)
    check_tree(case, mask, out, lse)


def test_tree_drafts_through_the_candidate_decode_kernel():
    # the prefix decode on the two-waves-per-SIMD candidate (MLA_DECODE_KERNEL
    # =w8: its bf16 partials and their merge), then the draft merge
    jobs, masks = [], []
    for dtype, P in (("bf16", 16), ("fp8_e4m3", 64)):
        case = make_case(kv_lens=[300, 8, 70, 1000], q_lens=[4, 8, 3, 0], seed=55, kv_dtype=dtype,
                         num_heads=16, page_size=P, sm_scale=1 / math.sqrt(192), max_q_len=8)
        mask = tree_masks(case.q_lens, case.max_q_len, "branch", seed=4)
        jobs.append((case, 6, 1, dict(tree_mask=mask, env_extra={
            "MLA_DECODE_KERNEL": "w8", "EMU_DMA_LAND": "issue", "EMU_SCHED": "drift"})))
        masks.append(mask)
    for (case, *_), mask, (out, lse, meta) in zip(jobs, masks, harness.run_many(jobs)):
        assert meta["num_partials"] > 0
        check_tree(case, mask, out, lse)


def test_tree_drafts_through_the_split_decode_kernel():
    # the prefix decode on the candidate whose pairs of waves share 32 rows
    # (MLA_DECODE_KERNEL=split: its bf16 partials and their merge), then the
    # draft merge, for both cache types and in two schedules
    jobs, masks = [], []
    for dtype, P in (("bf16", 16), ("fp8_e4m3", 64)):
        case = make_case(kv_lens=[300, 8, 70, 1000], q_lens=[4, 8, 3, 0], seed=56, kv_dtype=dtype,
                         num_heads=16, page_size=P, sm_scale=1 / math.sqrt(192), max_q_len=8)
        mask = tree_masks(case.q_lens, case.max_q_len, "branch", seed=5)
        for land, sched in (("issue", "drift"), ("wait", "lockstep")):
            jobs.append((case, 6, 1, dict(tree_mask=mask, env_extra={
                "MLA_DECODE_KERNEL": "split", "EMU_DMA_LAND": land, "EMU_SCHED": sched})))
            masks.append(mask)
    for (case, *_), mask, (out, lse, meta) in zip(jobs, masks, harness.run_many(jobs)):
        assert meta["num_partials"] > 0
        check_tree(case, mask, out, lse)

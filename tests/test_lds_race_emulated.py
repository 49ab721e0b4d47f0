"""LDS races in the decode kernels (and in the tree-draft merge and prefill
attention kernels), found by a happens-before detector in the lane-fiber
emulator (CPU only).

With EMU_LDS_RACE set, the LDS-trace build of the emulator
(tests/simt_emu/emu_runtime.cpp) treats each wave as one thread: a lane
carries a vector clock over the workgroup's waves, joined at every workgroup
barrier and handed over from lds_publish to the wait that sees the
published value.  Every traced LDS load and store, transposing read and
HBM -> LDS copy is checked per dword against the last write and the reads
since it, and a copy counts as written only once its wave has waited for it.
Two accesses of different waves that no barrier or counter orders are a
race even where the schedule that ran happened to put them in a harmless
order, so the check does not depend on the lockstep, drift or random
schedule finding the bad interleaving.

The checks: no decode kernel races on a case with several items per
workgroup, in any schedule, on seeded random shapes, or with tree-shaped
drafts (whose merge kernel shares the drafts' keys through LDS), and the
prefill attention kernel does not race either; each synchronisation step
taken out of a kernel (planted in a copy of the source, on the CPU only) is
reported, in the lockstep schedule, as the kind of race it opens; and the
library kernels' known restart-flag race (a wave sets the flag while another
still reads it in the same barrier interval) is reported whenever an item
restarts."""
import math
import os
import re
from concurrent.futures import ThreadPoolExecutor

import pytest

from tests.test_kernel_emulated import _available, _check, _rising_scores_case
from workloads import make_case

pytestmark = pytest.mark.skipif(not _available(), reason="host clang++ not available")

RACE = {"EMU_LDS_RACE": "1"}

# (MLA_DECODE_KERNEL, cache type, phases): the library's kernels (the 32-key
# pairs kernel is the bf16 one-phase default, the 16-key kernel serves e4m3
# and the phased plans) and the three candidates
KERNELS = [(None, "bf16", 1), (None, "bf16", 2), (None, "bf16", 4), (None, "fp8_e4m3", 1),
           (None, "fp8_e4m3", 4), ("qres", "fp8_e4m3", 1), ("w8", "bf16", 1),
           ("w8", "fp8_e4m3", 1), ("split", "bf16", 1), ("split", "fp8_e4m3", 1)]

SCHEDULES = {"lockstep": {}, "drift": {"EMU_SCHED": "drift"},
             "random": {"EMU_SCHED": "random", "EMU_SEED": "3"}}


@pytest.fixture(scope="module")
def binary():
    from tests.simt_emu import build as _b
    return _b.trace_binary()


def _case(kv_dtype):
    # several items per workgroup at 4 workgroups, two draft tokens, a
    # sequence shorter than a round and one spanning many pages
    return make_case(kv_lens=[700, 300, 130, 5], q_lens=[2, 1, 2, 1], seed=5, max_q_len=2,
                     kv_dtype=kv_dtype, sm_scale=1 / math.sqrt(192))


def _run(binary, kernel, kv_dtype, phases, env, nwg=4):
    from tests.simt_emu import harness
    extra = {**RACE, **env}
    if kernel:
        extra["MLA_DECODE_KERNEL"] = kernel
    case = _case(kv_dtype)
    out, lse, _ = harness.run(case, nwg, phases, env_extra=extra, binary=binary)
    _check(case, out, lse)


def test_decode_kernels_have_no_lds_race(binary):
    jobs = [(k, s) for k in KERNELS for s in SCHEDULES]

    def one(job):
        (kernel, kvd, phases), sched = job
        try:
            _run(binary, kernel, kvd, phases, SCHEDULES[sched])
            return None
        except (RuntimeError, AssertionError) as e:
            return job, str(e)[-600:]

    with ThreadPoolExecutor(max_workers=8) as ex:
        failures = [r for r in ex.map(one, jobs) if r]
    assert not failures, failures


def test_random_shapes_have_no_lds_race(binary):
    """Seeded random shapes through every decode kernel, race-checked: batch,
    heads, draft tokens, page size, lengths (at least the draft count),
    phase count, workgroup count and schedule drawn at random."""
    import numpy as np
    from tests.simt_emu import harness
    rng = np.random.default_rng(83)
    jobs = []
    for trial in range(40):
        kernel, kvd, phases = KERNELS[trial % len(KERNELS)]
        B, H, qmax = int(rng.integers(1, 5)), int(rng.choice([16, 32, 128])), int(rng.integers(1, 4))
        P = int(rng.choice([64, 256] if kvd == "fp8_e4m3" else [16, 64, 256]))
        ql = [int(x) for x in rng.integers(1, qmax + 1, B)]
        lens = [max(q, int(x)) for q, x in zip(ql, rng.integers(0, 900, B))]
        nwg = int(rng.integers(1, 12))
        nwg = max(phases, nwg - nwg % phases)
        sched = sorted(SCHEDULES)[trial % 3]
        case = make_case(kv_lens=lens, q_lens=ql, seed=trial, kv_dtype=kvd, max_q_len=qmax,
                         num_heads=H, page_size=P, sm_scale=1 / math.sqrt(192))
        env = {**RACE, **SCHEDULES[sched]}
        if kernel:
            env["MLA_DECODE_KERNEL"] = kernel
        jobs.append((case, nwg, phases, dict(env_extra=env, binary=binary)))
    for (case, *_), (out, lse, _meta) in zip(jobs, harness.run_many(jobs, workers=8)):
        _check(case, out, lse)


# Synchronisation steps taken out, one at a time: (source file, text, its
# replacement, cache type, the race the detector must report, and the
# MLA_DECODE_KERNEL value that runs it where the library's default does not).
PLANTS = {
    # the default bf16 kernel's per-round barrier: a wave reads tiles that
    # other waves copied, with no barrier after their waits for the copies
    "pairs_barrier": ("decode_kernel.hip",
                      "vm_wait_rounds<KVD>(ahead);\n"
                      "        barrier();   // tiles of round j come from all waves",
                      "vm_wait_rounds<KVD>(ahead);", "bf16", "read after write"),
    # the 16-key kernel's (the e4m3 default)
    "e4m3_barrier": ("decode_kernel.hip",
                     "{\n          barrier();   // tiles of round j come from all waves", "{",
                     "fp8_e4m3", "read after write"),
    # the same step in the Q-resident rebuild, which is that source compiled
    # with Q forced resident
    "qres_barrier": ("decode_kernel.hip",
                     "{\n          barrier();   // tiles of round j come from all waves", "{",
                     "fp8_e4m3", "read after write", "qres"),
    "w8_barrier": ("decode_w8_kernel.hip", "barrier();   // tiles of round j come from all waves",
                   "/* removed */", "bf16", "read after write", "w8"),
    # the 16-rows-per-wave candidate's e4m3 pipeline: the barrier after a
    # pair's widening, and the wait for the next round's copies
    "w8_f8_barrier": ("decode_w8_kernel.hip",
                      "barrier();   // pair p widened by all waves; for odd p, round j + 1 copied",
                      "/* removed */", "fp8_e4m3", "read after write", "w8"),
    "w8_f8_wait": ("decode_w8_kernel.hip", "if (pp == 1) MLA_VM_WAIT(0);", "/* removed */",
                   "fp8_e4m3", "read of a copy in flight", "w8"),
    # the split candidate: its round barrier, its wait for a round's copies,
    # its partner's round counter and the barrier that closes an item
    "split_barrier": ("decode_split_kernel.hip",
                      "barrier();   // round j from all waves; round j - 1 and its exchange done",
                      "/* removed */", "bf16", "read after write"),
    "split_copy_wait": ("decode_split_kernel.hip", "if (j + 1 < nrounds) MLA_VM_WAIT(4);",
                        "if (j + 1 < nrounds) MLA_VM_WAIT(8);", "bf16", "read of a copy in flight"),
    "split_partner_wait": ("decode_split_kernel.hip", "lds_wait_at_least(flag_par, seq);",
                           "/* removed */", "bf16", "read after write"),
    "split_item_barrier": ("decode_split_kernel.hip",
                           "    // item's prologue refills them\n    barrier();",
                           "    // item's prologue refills them", "bf16", "write after read"),
    # its e4m3 pipeline: the round barrier, the wait for the round about to
    # be widened, and the prologue's wait for round 0
    "split_f8_barrier": ("decode_split_kernel.hip",
                         "barrier();   // round p widened and round p + 1 copied by all waves; "
                         "round p - 1 done", "/* removed */", "fp8_e4m3", "write after read"),
    "split_f8_copy_wait": ("decode_split_kernel.hip", "if (p + 2 < nrounds) MLA_VM_WAIT(2);",
                           "if (p + 2 < nrounds) MLA_VM_WAIT(5);", "fp8_e4m3",
                           "read of a copy in flight"),
    "split_f8_first_wait": ("decode_split_kernel.hip",
                            "MLA_VM_WAIT(0);   // this wave's copies of round 0 (and its Q loads)",
                            "/* removed */", "fp8_e4m3", "read of a copy in flight"),
}


@pytest.fixture(scope="module")
def planted():
    """{plant: emulator binary}, built four at a time (each recompiles only
    the units its patched file enters)."""
    from tests.simt_emu import build as _b

    def one(name):
        fname, old, new = PLANTS[name][:3]
        src = open(os.path.join(_b.CSRC, fname)).read()
        assert src.count(old) == 1, name
        return _b.build(tag="race_" + name, lds_trace=True, patches={fname: [(old, new)]})

    names = sorted(PLANTS)
    _b.trace_binary()   # the base the variants link against, brought up to date once
    with ThreadPoolExecutor(max_workers=4) as ex:
        return dict(zip(names, ex.map(one, names)))


@pytest.mark.parametrize("plant", sorted(PLANTS))
def test_detector_reports_each_planted_mistake(planted, plant):
    fname, _old, _new, kvd, kind, *kernel = PLANTS[plant]
    kernel = kernel[0] if kernel else {"decode_split_kernel.hip": "split"}.get(fname)
    with pytest.raises(RuntimeError, match=re.escape(f"LDS race ({kind})")):
        _run(planted[plant], kernel, kvd, 1, {})


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8_e4m3"])
def test_detector_reports_the_library_restart_flag_race(binary, kv_dtype):
    # Scores that restart the item every 32 keys: a wave that overshoots sets
    # the library kernels' single restart flag while other waves of the same
    # barrier interval still read it (the race the drift schedule turns into
    # a barrier deadlock); the detector names the flag's word in any
    # schedule (152576 is that word's offset, kFlagOff in decode_kernel.hip).
    # The candidates rescale instead and stay race-free.
    from tests.simt_emu import harness
    case = _rising_scores_case(kv_dtype, L=160)
    with pytest.raises(RuntimeError, match=r"LDS race \(write after read\) at LDS byte 152576"):
        harness.run(case, 1, 1, env_extra=RACE, binary=binary)
    for kernel in ("w8", "split"):
        out, lse, _ = harness.run(case, 1, 1, env_extra={**RACE, "MLA_DECODE_KERNEL": kernel},
                                  binary=binary)
        _check(case, out, lse)


def test_fifth_fault_plan_is_race_free():
    # The plan of the fifth faulting GPU run (the library's planner with a
    # per-piece charge of one round and one-round pieces: one workgroup takes
    # two one-round items back to back), built for the emulator only, in the
    # e4m3 case and page relayout it faulted on: no LDS race in any schedule
    # or copy-landing mode, so the kernel's LDS protocol does not explain it.
    from tests.simt_emu import build as _b, harness
    from tests.test_kernel_emulated import _plan_items, _relayout
    binary = _b.build(tag="race_min_piece_1", lds_trace=True, patches={"plan_core.h": [
        ("constexpr int kMinPieceRounds = 2;", "constexpr int kMinPieceRounds = 1;")]})
    case = make_case(kv_lens=[700, 64, 1234], q_lens=[2, 1, 1], kv_dtype="fp8_e4m3", seed=22,
                     sm_scale=1 / math.sqrt(192))
    jobs = []
    for c in (case, _relayout(case, 5)):
        for sched in SCHEDULES.values():
            for land in ("wait", "issue"):
                env = {**RACE, **sched, "MLA_ITEM_COST_ROUNDS": "1", "EMU_DMA_LAND": land}
                jobs.append((c, 16, 1, dict(binary=binary, env_extra=env, want_plan=True)))
    for (c, *_), (out, lse, meta) in zip(jobs, harness.run_many(jobs, workers=8)):
        assert sum(len(w) == 2 for w in _plan_items(meta["plan"])) == 1
        _check(c, out, lse)


def test_tree_drafts_have_no_lds_race(binary):
    # the tree-draft path (a non-causal decode of the prefix, then
    # mla_tree_attend, whose workgroups share the drafts' keys through LDS)
    # with every mask kind, both cache types and each decode kernel that
    # takes it, race-checked
    from tests.simt_emu import harness
    from tests.test_tree_emulated import check_tree
    from tests.tree_cases import tree_masks
    jobs = []
    for n, kind in enumerate(("causal", "diag", "branch", "random", "none")):
        kvd = ("bf16", "fp8_e4m3")[n % 2]
        case = make_case(kv_lens=[300, 8, 70, 4, 1000], q_lens=[4, 8, 3, 4, 0], seed=51,
                         num_heads=16, page_size=64, kv_dtype=kvd, sm_scale=1 / math.sqrt(192),
                         max_q_len=8)
        mask = tree_masks(case.q_lens, case.max_q_len, kind, seed=2)
        for kernel in (None, "w8", "split"):
            env = dict(RACE, **({"MLA_DECODE_KERNEL": kernel} if kernel else {}))
            jobs.append(((case, mask), 6, 1, dict(tree_mask=mask, env_extra=env, binary=binary)))
    runs = harness.run_many([(c, n, p, kw) for (c, _m), n, p, kw in jobs], workers=8)
    for ((case, mask), *_), (out, lse, _meta) in zip(jobs, runs):
        check_tree(case, mask, out, lse)


def test_detector_reports_a_missing_tree_barrier():
    # the tree merge kernel with its barrier after the drafts' keys are
    # written taken out (on the CPU only): a wave reads keys another wave
    # has yet to write
    from tests.simt_emu import build as _b, harness
    from tests.tree_cases import tree_masks
    old = "    dst[1] = v1;\n  }\n  __syncthreads();"
    assert open(os.path.join(_b.CSRC, "tree_kernel.hip")).read().count(old) == 1
    binary = _b.build(tag="race_tree_barrier", lds_trace=True,
                      patches={"tree_kernel.hip": [(old, "    dst[1] = v1;\n  }")]})
    case = make_case(kv_lens=[300, 8, 70, 4, 1000], q_lens=[4, 8, 3, 4, 0], seed=51,
                     num_heads=16, page_size=64, sm_scale=1 / math.sqrt(192), max_q_len=8)
    mask = tree_masks(case.q_lens, case.max_q_len, "branch", seed=2)
    with pytest.raises(RuntimeError, match=r"LDS race \(write after read\) at shared address"):
        harness.run(case, 6, 1, tree_mask=mask, env_extra=RACE, binary=binary)


def _prefill(binary):
    from oracle import prefill_ref
    from tests.prefill_cases import check_attention, check_quantized
    from tests.simt_emu import harness
    from workloads.prefill import make_prefill_case
    case = make_prefill_case(seqlens=[300, 1, 5, 129], num_heads=2, seed=71)
    got = harness.run_prefill(case, prefill_ref.num_blocks(case.seqlens), env_extra=RACE,
                              binary=binary)
    check_attention(case, got["o"], got["lse"], quantized=check_quantized(case, got))


def test_prefill_attention_has_no_lds_race(binary):
    # the quantized prefill's attention kernel, whose waves share each key
    # block's INT8 keys, e4m3 values and value exponents through LDS
    _prefill(binary)


def test_detector_reports_a_missing_prefill_barrier():
    # its barrier between writing a key block and reading it taken out (on
    # the CPU only)
    from tests.simt_emu import build as _b
    old = "    store_block<kThreads>(regs, ktile, vtile, vexp);\n    const float kscale = regs.ks;\n" \
          "    __syncthreads();"
    new = "    store_block<kThreads>(regs, ktile, vtile, vexp);\n    const float kscale = regs.ks;"
    assert open(os.path.join(_b.CSRC, "prefill_attn_kernel.hip")).read().count(old) == 1
    binary = _b.build(tag="race_prefill_barrier", lds_trace=True,
                      patches={"prefill_attn_kernel.hip": [(old, new)]})
    with pytest.raises(RuntimeError, match=r"LDS race \((read after write|write after read)\)"):
        _prefill(binary)

"""GPU parity of the HIP path (through the C ABI) against the float64 oracle.

Bars (from the problem statement): bf16 cache max-abs <= 2e-2 and rel-L2 <= 5e-3;
fp8-e4m3 cache 6e-2 and 2e-2; LSE |diff| <= 1e-3 (a bar of this library's own: the
problem statement gives none for LSE);
indexing exact (bitwise-identical output under page relayout for a fixed plan).
"""
import math
import os

import numpy as np
import pytest

import oracle
from workloads import MLACase, make_case, workload

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import mla_paged_decode_absorbed_amd as mla  # noqa: E402

TOL = {"bf16": (2e-2, 5e-3), "fp8_e4m3": (6e-2, 2e-2)}
LSE_TOL = 1e-3
DEV = "cuda"
SENTINEL = 0x7FC1   # bf16 NaN pattern pre-filled into O; padded rows must keep it


def to_dev(case: MLACase, block_table=None):
    q = torch.from_numpy(case.q.view(np.int16)).view(torch.bfloat16).to(DEV)
    if case.kv_dtype == "bf16":
        kv = torch.from_numpy(case.kv.view(np.int16)).view(torch.bfloat16).to(DEV)
    else:
        kv = torch.from_numpy(case.kv).to(DEV)
    sc = None if case.kv_scale is None else torch.from_numpy(case.kv_scale).to(DEV)
    bt = torch.from_numpy(case.block_table if block_table is None else block_table).to(DEV)
    kvl = torch.from_numpy(case.kv_lens).to(DEV)
    ql = torch.from_numpy(case.q_lens).to(DEV)
    return q, kv, sc, bt, kvl, ql


def shape_of(case: MLACase, block_table=None):
    bt = case.block_table if block_table is None else block_table
    return mla.Shape.make(batch=case.batch, num_heads=case.num_heads, max_q_len=case.max_q_len,
                          page_size=case.page_size, num_pages=case.num_pages,
                          max_pages_per_seq=bt.shape[1],
                          kv_dtype=mla.KV_BF16 if case.kv_dtype == "bf16" else mla.KV_FP8_E4M3,
                          causal=case.causal)


def make_plan(shape, case, num_workgroups=None, phases=None):
    """Host plan; ``phases`` forces the workgroup-group size (MLA_PHASES)."""
    old = os.environ.get("MLA_PHASES")
    try:
        if phases is not None:
            os.environ["MLA_PHASES"] = str(phases)
        pl = mla.plan(shape, case.kv_lens, case.q_lens, num_workgroups=num_workgroups)
    finally:
        if phases is not None:
            if old is None:
                del os.environ["MLA_PHASES"]
            else:
                os.environ["MLA_PHASES"] = old
    if phases is not None:
        assert pl.phases == phases
    return pl


def run_gpu(case: MLACase, num_workgroups=None, block_table=None, pl=None, repeats=1,
            phases=None):
    shape = shape_of(case, block_table)
    if pl is None:
        pl = make_plan(shape, case, num_workgroups, phases)
    q, kv, sc, bt, kvl, ql = to_dev(case, block_table)
    outs = []
    for _ in range(repeats):
        out = torch.full((case.batch, case.max_q_len, case.num_heads, 512), 0, dtype=torch.int16,
                         device=DEV)
        out.fill_(SENTINEL)
        out = out.view(torch.bfloat16)
        lse = torch.full((case.batch, case.max_q_len, case.num_heads), 12345.0,
                         dtype=torch.float32, device=DEV)
        mla.decode(shape, pl, q, kv, bt, kvl, ql, case.sm_scale, kv_scale=sc, out=out, lse=lse)
        torch.cuda.synchronize()
        outs.append((out, lse))
    return outs if repeats > 1 else outs[0], pl


def as_f64(out, lse):
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def check(case: MLACase, out, lse, seqs=None, tol=None):
    seqs = list(range(case.batch)) if seqs is None else list(seqs)
    O, L = oracle.mla_decode_ref(case, seqs=seqs)
    o, l = as_f64(out, lse)
    mabs, mrel = tol or TOL[case.kv_dtype]
    num = den = 0.0
    worst = 0.0
    for b in seqs:
        qb = int(case.q_lens[b])
        if qb == 0:
            continue
        d = o[b, :qb] - O[b, :qb]
        assert np.all(np.isfinite(o[b, :qb])), f"non-finite output in sequence {b}"
        worst = max(worst, float(np.abs(d).max()))
        num += float((d ** 2).sum())
        den += float((O[b, :qb] ** 2).sum())
        dl = np.abs(l[b, :qb] - L[b, :qb])
        assert dl.max() <= LSE_TOL, f"LSE error {dl.max():.3g} in sequence {b}"
    rel = math.sqrt(num / max(den, 1e-300))
    assert worst <= mabs, f"max-abs {worst:.4g} > {mabs}"
    assert rel <= mrel, f"rel-L2 {rel:.4g} > {mrel}"
    # padded rows (t >= q_len) are neither read nor written
    raw = out.view(torch.int16).cpu().numpy()
    for b in seqs:
        qb = int(case.q_lens[b])
        if qb < case.max_q_len:
            assert np.all(raw[b, qb:] == SENTINEL), f"padded rows of sequence {b} were written"
            assert np.all(lse[b, qb:].cpu().numpy() == 12345.0)
    return worst, rel


# ---------------------------------------------------------------- small, exhaustive

PHASES = [1, 2, 4]


@pytest.mark.parametrize("phases", PHASES)
@pytest.mark.parametrize("kv_lens", [[1], [15, 16, 17], [63, 64, 65, 127, 128, 129], [4097]])
def test_bf16_q1_edge_lengths(kv_lens, phases):
    case = make_case(kv_lens=kv_lens, seed=11, sm_scale=1 / math.sqrt(192))
    (out, lse), _ = run_gpu(case, phases=phases)
    check(case, out, lse)


@pytest.mark.parametrize("phases", PHASES)
@pytest.mark.parametrize("kv_lens", [[2, 3], [33, 64, 65], [300, 1000]])
def test_bf16_q2_causal(kv_lens, phases):
    case = make_case(kv_lens=kv_lens, q_lens=[2] * len(kv_lens), seed=12,
                     sm_scale=1 / math.sqrt(192))
    (out, lse), _ = run_gpu(case, phases=phases)
    check(case, out, lse)


@pytest.mark.parametrize("phases", PHASES)
def test_bf16_mixed_q_lens_and_empty_sequence(phases):
    case = make_case(kv_lens=[70, 2, 900, 5, 129], q_lens=[1, 2, 2, 0, 1], max_q_len=2, seed=13,
                     sm_scale=1 / math.sqrt(192))
    (out, lse), _ = run_gpu(case, phases=phases)
    check(case, out, lse)


@pytest.mark.parametrize("phases", [1, 4])
@pytest.mark.parametrize("H,q", [(16, 1), (16, 2), (64, 2), (128, 3), (32, 4), (128, 4),
                                 (128, 5)])
def test_head_counts_and_longer_drafts(H, q, phases):
    case = make_case(kv_lens=[97, 640, max(4, q)], q_lens=[q, q, q], num_heads=H, seed=14,
                     sm_scale=1 / math.sqrt(192))
    (out, lse), _ = run_gpu(case, phases=phases)
    check(case, out, lse)


@pytest.mark.parametrize("phases", [1, 4])
@pytest.mark.parametrize("H", [16, 128])
def test_max_draft_length(H, phases):
    # MLA_MAX_Q_LEN = 8 query tokens per sequence: up to 8 row blocks of 128
    case = make_case(kv_lens=[40, 600, 8], q_lens=[8, 8, 8], num_heads=H, seed=15,
                     sm_scale=1 / math.sqrt(192))
    (out, lse), _ = run_gpu(case, num_workgroups=16, phases=phases)
    check(case, out, lse)


def test_non_causal_q2():
    case = make_case(kv_lens=[50, 333], q_lens=[2, 2], causal=False, seed=15,
                     sm_scale=1 / math.sqrt(192))
    (out, lse), _ = run_gpu(case)
    check(case, out, lse)


@pytest.mark.parametrize("P", [16, 32, 128, 256])
def test_bf16_page_sizes(P):
    case = make_case(kv_lens=[1, 255, 700], page_size=P, seed=16, sm_scale=1 / math.sqrt(192))
    (out, lse), _ = run_gpu(case)
    check(case, out, lse)


@pytest.mark.parametrize("phases", PHASES)
@pytest.mark.parametrize("nwg", [1, 4, 8, 64, 256, 1000])
def test_forced_split_counts(nwg, phases):
    if nwg % phases:
        pytest.skip("workgroup count not a multiple of the group size")
    case = make_case(kv_lens=[3000, 700, 65, 1800], q_lens=[1, 2, 1, 2], seed=17,
                     sm_scale=1 / math.sqrt(192))
    (out, lse), pl = run_gpu(case, num_workgroups=nwg, phases=phases)
    check(case, out, lse)
    if nwg >= 64 * phases:
        assert pl.info.num_combine > 0


@pytest.mark.parametrize("phases", PHASES)
def test_peaky_softmax(phases):
    # scores spread over hundreds of units: later tiles overshoot the first
    # tile's reference max and restart their item
    case = make_case(kv_lens=[2000, 513], q_lens=[1, 2], seed=18, q_std=8.0,
                     sm_scale=1 / math.sqrt(192))
    (out, lse), _ = run_gpu(case, phases=phases)
    check(case, out, lse)


@pytest.mark.parametrize("phases", PHASES)
def test_late_dominant_key(phases):
    case = make_case(kv_lens=[1500], q_lens=[1], seed=19, sm_scale=1 / math.sqrt(192))
    q = oracle.decode_bf16(case.q[0, 0])
    # overwrite cached token 1400 with a copy of head 0's query: its score is
    # over 50 (log2 units) above the first tile's maximum, past the 32 that
    # makes the kernel restart the item with a raised reference max
    L = 1400
    page, slot = case.block_table[0, L // 64], L % 64
    import torch as _t
    v = _t.from_numpy(q[0].astype(np.float32)).to(_t.bfloat16).view(_t.int16).numpy()
    case.kv[page, slot] = v.view(np.uint16)
    (out, lse), _ = run_gpu(case, num_workgroups=phases, phases=phases)
    check(case, out, lse)


@pytest.mark.parametrize("phases", PHASES)
def test_fp8_small(phases):
    case = make_case(kv_lens=[1, 64, 65, 1000, 3000], q_lens=[1, 1, 2, 2, 1], kv_dtype="fp8_e4m3",
                     seed=20, sm_scale=1 / math.sqrt(192))
    (out, lse), _ = run_gpu(case, phases=phases)
    check(case, out, lse)


@pytest.mark.parametrize("nwg", [3, 256])
def test_fp8_splits(nwg):
    case = make_case(kv_lens=[5000, 129], kv_dtype="fp8_e4m3", seed=21,
                     sm_scale=1 / math.sqrt(192))
    (out, lse), _ = run_gpu(case, num_workgroups=nwg)
    check(case, out, lse)


# ---------------------------------------------------------------- indexing exactness

def _relayout(case, seed):
    """Same logical cache, new random page placement (fresh pool, poisoned)."""
    rng = np.random.default_rng(seed)
    perm = rng.permutation(case.num_pages).astype(np.int32)
    kv = np.empty_like(case.kv)
    kv[perm] = case.kv
    sc = None
    if case.kv_scale is not None:
        sc = np.empty_like(case.kv_scale)
        sc[perm] = case.kv_scale
    bt = np.where(case.block_table >= 0, perm[np.maximum(case.block_table, 0)], -1).astype(np.int32)
    return MLACase(**{**case.__dict__, "kv": kv, "kv_scale": sc, "block_table": bt})


@pytest.mark.parametrize("phases", [1, 4])
@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8_e4m3"])
def test_page_relayout_is_bitwise_identical(kv_dtype, phases):
    case = make_case(kv_lens=[700, 64, 1234], q_lens=[2, 1, 1], kv_dtype=kv_dtype, seed=22,
                     sm_scale=1 / math.sqrt(192))
    (o1, l1), pl = run_gpu(case, num_workgroups=16, phases=phases)
    c2 = _relayout(case, 5)
    (o2, l2), _ = run_gpu(c2, pl=pl)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


def test_unused_block_table_entries_never_read():
    case = make_case(kv_lens=[100, 40], seed=23, extra_pages_per_seq=3,
                     sm_scale=1 / math.sqrt(192))
    bt = case.block_table.copy()
    bt[bt < 0] = np.iinfo(np.int32).max
    (out, lse), _ = run_gpu(case, block_table=bt)
    check(case, out, lse)


@pytest.mark.parametrize("phases", PHASES)
def test_repeat_runs_bitwise_equal(phases):
    case = make_case(kv_lens=[2500, 900, 33], q_lens=[2, 1, 2], seed=24,
                     sm_scale=1 / math.sqrt(192))
    runs, _ = run_gpu(case, num_workgroups=64, repeats=20, phases=phases)
    o0, l0 = runs[0]
    for o, l in runs[1:]:
        assert torch.equal(o.view(torch.int16), o0.view(torch.int16)) and torch.equal(l, l0)


# ---------------------------------------------------------------- standalone combine

def test_combine_kernel_matches_combine_ref():
    case = make_case(kv_lens=[3000, 2500], q_lens=[2, 1], seed=25, sm_scale=1 / math.sqrt(192))
    shape = shape_of(case)
    pl = mla.plan(shape, case.kv_lens, case.q_lens, num_workgroups=64)
    assert pl.info.num_combine > 0
    rng = np.random.default_rng(0)
    P = pl.info.num_partials
    po = rng.standard_normal((P, 128, 512)).astype(np.float32)
    plse = (rng.standard_normal((P, 128)) * 3).astype(np.float32)
    # some partials empty (LSE = -inf, O = NaN garbage that must be ignored)
    plse[::5, ::7] = -np.inf
    po[::5, ::7] = np.nan
    ws = mla.alloc_workspace(pl)
    base = ws.view(torch.float32)
    base[: P * 128 * 512].copy_(torch.from_numpy(po.reshape(-1)))
    base[P * 128 * 512: P * 128 * 512 + P * 128].copy_(torch.from_numpy(plse.reshape(-1)))
    out = torch.zeros((case.batch, 2, case.num_heads, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.zeros((case.batch, 2, case.num_heads), dtype=torch.float32, device=DEV)
    ql = torch.from_numpy(case.q_lens).to(DEV)
    mla.combine(shape, pl, ws, ql, out, lse)
    torch.cuda.synchronize()
    o, l = as_f64(out, lse)
    for b, row0, first, n in pl.combine_entries():
        Oc, Lc = oracle.combine_ref(po[first:first + n], plse[first:first + n])
        rows = min(128, int(case.q_lens[b]) * case.num_heads - int(row0))
        for r in range(rows):
            row = int(row0) + r
            t, h = divmod(row, case.num_heads)
            if np.isneginf(Lc[r]):
                assert np.isneginf(l[b, t, h]) and np.all(o[b, t, h] == 0)
                continue
            assert abs(l[b, t, h] - Lc[r]) <= 1e-4 * max(1.0, abs(Lc[r]))
            # fp32 merge, then one bf16 rounding: at most 2^-9 of the row's
            # largest value, so 4e-3 of it leaves a factor of two
            err = np.abs(o[b, t, h] - Oc[r]).max()
            assert err <= 4e-3 * np.abs(Oc[r]).max()


# ---------------------------------------------------------------- full-size workloads
# The four workloads at their full sizes, in the launch configuration bench.py
# times (one workgroup per CU): every sequence against the float64 oracle,
# max-abs and rel-L2 over the whole output tensor (about 1 s to 15 s of
# oracle time each on 16 host threads).

FULL = ["v3_decode_bf16", "mtp_verify_bf16", "long_ctx_fp8", "ragged_serving_bf16"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_workloads(name):
    case = workload(name)
    (out, lse), pl = run_gpu(case)
    print(f"{name}: workgroups {pl.info.num_workgroups} items {pl.info.num_items} "
          f"partials {pl.info.num_partials}", flush=True)
    worst, rel = check(case, out, lse)
    print(f"{name}: all {case.batch} sequences: max-abs {worst:.3g} rel-L2 {rel:.3g}",
          flush=True)

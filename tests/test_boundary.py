"""C-ABI boundary checks that need no GPU: the library loads and exports its
symbols, the planner's schedule is a valid partition, and argument validation
returns the documented status codes before any device work."""
import ctypes
import subprocess

import numpy as np
import pytest

import mla_paged_decode_absorbed_amd as mla

HEADER = "include/mla_decode.h"


@pytest.fixture(scope="module")
def lib():
    return mla.load_library()


def test_exports_every_declared_symbol(lib):
    import os, re
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    decl = open(os.path.join(root, HEADER)).read()
    names = set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\*?\s+\*?(mla_[a-z_0-9]+)\(", decl, re.M))
    assert names == set(mla.EXPORTED_SYMBOLS)
    dyn = subprocess.run(["nm", "-D", "--defined-only", mla.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    for n in names:
        assert re.search(rf"\bT {n}$", dyn, re.M), n
        assert getattr(lib, n) is not None


def test_version_and_status_strings(lib):
    assert lib.mla_abi_version() == 2
    for st in range(9):
        assert len(mla.status_string(st)) >= 2
    assert mla.status_string(99) == "unknown status"


def _shape(B=4, H=128, qmax=1, P=64, pages=1000, maxp=200, kvd=mla.KV_BF16, causal=True, **kw):
    return mla.Shape.make(batch=B, num_heads=H, max_q_len=qmax, page_size=P, num_pages=pages,
                          max_pages_per_seq=maxp, kv_dtype=kvd, causal=causal, **kw)


def _check_partition(shape, pl, kv_lens, q_lens):
    """Every (sequence, query row, key round) is covered by exactly one item; the
    pieces of a 128-row unit are contiguous and ordered, split at round
    boundaries; the workgroups of one piece share its key range and cover
    disjoint row slices; slots/combine agree."""
    R_TOK = 64
    items = pl.items()
    ws = pl.wg_start()
    PH = pl.phases
    assert PH in (1, 2, 4)
    assert ws[0] == 0 and ws[-1] == len(items) and np.all(np.diff(ws) >= 0)
    H = shape.num_heads
    want = {}
    for b in range(shape.batch):
        q = shape.max_q_len if q_lens is None else int(q_lens[b])
        for r0 in range(0, q * H, 128):
            want[(b, r0)] = (int(kv_lens[b]), min(128, q * H - r0))
    got = {}
    for g in range(pl.info.num_workgroups):
        for it in items[ws[g]:ws[g + 1]]:
            b, row0, k0, k1, slot, off = map(int, it)
            assert off % (128 // PH) == 0 and 0 <= off < 128
            # the workgroups of one piece are consecutive and start on a multiple of PH
            assert g % PH == off // (128 // PH)
            got.setdefault((b, row0 - off), []).append((k0, k1, slot, off, g // PH))
    assert set(got) == set(want)
    comb = {(int(c[0]), int(c[1])): (int(c[2]), int(c[3])) for c in pl.combine_entries()}
    used_slots = []
    for key, parts in got.items():
        L, rows = want[key]
        n_sub = -(-rows // (128 // PH))
        pieces = {}
        for k0, k1, slot, off, proc in parts:
            pieces.setdefault((k0, k1, slot), []).append((off, proc))
        for (k0, k1, slot), subs in pieces.items():
            offs = sorted(o for o, _ in subs)
            assert offs == [i * (128 // PH) for i in range(n_sub)]
            assert len({p for _, p in subs}) == 1     # one processor per piece
        ranges = sorted(pieces)
        assert ranges[0][0] == 0 and ranges[-1][1] == L
        for (a0, a1, _), (b0, b1, _) in zip(ranges, ranges[1:]):
            assert a1 == b0 and a0 < a1 and b0 % R_TOK == 0
        if len(ranges) == 1:
            assert ranges[0][2] == -1 and key not in comb
        else:
            first, n = comb[key]
            assert n == len(ranges)
            assert [p[2] for p in ranges] == list(range(first, first + n))
            used_slots += [p[2] for p in ranges]
    # the image's own counts (a fixed-shape plan's info holds launch bounds)
    assert sorted(used_slots) == list(range(int(pl.host[5])))
    assert int(pl.host[4]) == len(comb)
    return items


@pytest.mark.parametrize("seed,B,qmax,lo,hi,kvd", [
    (0, 64, 1, 1024, 4096, mla.KV_BF16),
    (1, 128, 2, 512, 8192, mla.KV_BF16),
    (2, 16, 1, 16384, 32768, mla.KV_FP8_E4M3),
    (3, 7, 2, 2, 300, mla.KV_BF16),
    (4, 1, 1, 1, 1, mla.KV_BF16),
    (5, 300, 1, 64, 200, mla.KV_BF16),
])
def test_plan_partitions_and_balances(seed, B, qmax, lo, hi, kvd):
    rng = np.random.default_rng(seed)
    kv = rng.integers(lo, hi, size=B, endpoint=True).astype(np.int32)
    ql = rng.integers(1, qmax, size=B, endpoint=True).astype(np.int32) if qmax > 1 else None
    kv = np.maximum(kv, 2 if qmax > 1 else 1).astype(np.int32)
    maxp = int((kv.max() + 63) // 64)
    shape = _shape(B=B, qmax=qmax, pages=int(((kv + 63) // 64).sum()), maxp=maxp, kvd=kvd)
    pl = mla.plan(shape, kv, ql, num_workgroups=256, upload=False)
    items = _check_partition(shape, pl, kv, ql)
    assert (pl.info.num_partials, pl.info.num_combine) == (int(pl.host[5]), int(pl.host[4]))
    # balance: per-workgroup round cost within one item cost (+ a cut's slack) of the mean
    ws = pl.wg_start()
    cost = [sum((int(it[3]) - int(it[2]) + 63) // 64 + 2 for it in items[ws[g]:ws[g + 1]])
            for g in range(pl.info.num_workgroups)]
    mean = sum(cost) / len(cost)
    assert max(cost) <= np.ceil(mean) + 2 + 2
    assert pl.info.num_workgroups <= 256
    assert pl.info.workspace_bytes <= mla.load_library().mla_workspace_bytes_bound(
        ctypes.byref(shape), 256)


def test_plan_deterministic_and_mixed_q_lens():
    kv = np.array([5, 4000, 70, 1, 9000], np.int32)
    ql = np.array([2, 1, 2, 0, 1], np.int32)
    shape = _shape(B=5, qmax=2, maxp=200)
    a = mla.plan(shape, kv, ql, num_workgroups=32, upload=False)
    b = mla.plan(shape, kv, ql, num_workgroups=32, upload=False)
    assert np.array_equal(a.host, b.host)
    items = _check_partition(shape, a, kv, ql)
    assert not any(int(it[0]) == 3 for it in items)   # q_len 0 -> no work


def test_non_causal_zero_length_gets_an_item():
    shape = _shape(B=2, causal=False)
    pl = mla.plan(shape, np.array([0, 100], np.int32), num_workgroups=8, upload=False)
    items = pl.items()
    assert any(int(it[0]) == 0 and int(it[2]) == 0 and int(it[3]) == 0 for it in items)


@pytest.mark.parametrize("kw,kv,ql,status", [
    (dict(d_latent=256), [10], None, 3),
    (dict(P=8), [10], None, 3),
    (dict(P=48), [10], None, 3),
    (dict(P=32, kvd=mla.KV_FP8_E4M3), [10], None, 3),
    (dict(kvd=7), [10], None, 3),
    (dict(qmax=9), [10], None, 3),
    (dict(H=0), [10], None, 2),
    (dict(maxp=1), [65], None, 2),            # kv_len beyond the block-table capacity
    (dict(qmax=2), [1], [2], 2),              # causal: kv_len < q_len
    (dict(qmax=2), [5], [3], 2),              # q_len > max_q_len
    (dict(), [-1], None, 2),
])
def test_plan_rejects(kw, kv, ql, status):
    shape = _shape(B=1, **kw)
    with pytest.raises(mla.MLAError) as e:
        mla.plan(shape, np.array(kv, np.int32), None if ql is None else np.array(ql, np.int32),
                 num_workgroups=8, upload=False)
    assert e.value.status == status


def test_plan_buffer_too_small(lib):
    shape = _shape(B=3)
    kv = np.array([100, 200, 300], np.int32)
    buf = np.zeros(8, np.int32)
    info = mla.PlanInfo()
    st = lib.mla_decode_plan(ctypes.byref(shape), kv.ctypes.data, None, 8, buf.ctypes.data,
                             buf.nbytes, ctypes.byref(info))
    assert st == 6
    st = lib.mla_decode_plan(None, kv.ctypes.data, None, 8, buf.ctypes.data, buf.nbytes,
                             ctypes.byref(info))
    assert st == 1


class _FakeTensor:
    def __init__(self, addr):
        self.addr = addr

    def data_ptr(self):
        return self.addr


def test_fwd_and_combine_validate_before_any_launch(lib):
    shape = _shape(B=2)
    pl = mla.plan(shape, np.array([100, 3000], np.int32), num_workgroups=64, upload=False)
    info = pl.info
    A = 0x10000   # aligned fake device addresses; never dereferenced on these paths
    args = dict(plan=A, q=A, kv=A, scale=None, bt=A, kvl=A, ql=None, o=A, lse=A, ws=A)

    def fwd(**over):
        a = {**args, **over}
        return lib.mla_decode_fwd(ctypes.byref(shape), ctypes.byref(info), a["plan"], a["q"],
                                  a["kv"], a["scale"], a["bt"], a["kvl"], a["ql"], 0.07, a["o"],
                                  a["lse"], a["ws"], a.get("wsb", 0), None)

    assert fwd(q=None) == 1
    assert fwd(o=None) == 1
    assert fwd(q=A + 8) == 4
    assert fwd(ws=A + 16, wsb=1 << 40) == 4 if info.num_partials else True
    if info.num_partials:
        assert fwd(wsb=16) == 5
    bad = mla.PlanInfo.from_buffer_copy(info)
    bad.tile_tokens = 64
    assert lib.mla_decode_fwd(ctypes.byref(shape), ctypes.byref(bad), A, A, A, None, A, A, None,
                              0.07, A, A, A, 1 << 40, None) == 7
    bad = mla.PlanInfo.from_buffer_copy(info)
    bad.phases = 3
    assert lib.mla_decode_fwd(ctypes.byref(shape), ctypes.byref(bad), A, A, A, None, A, A, None,
                              0.07, A, A, A, 1 << 40, None) == 7
    fp8 = _shape(B=2, kvd=mla.KV_FP8_E4M3)
    pl8 = mla.plan(fp8, np.array([100, 3000], np.int32), num_workgroups=64, upload=False)
    assert lib.mla_decode_fwd(ctypes.byref(fp8), ctypes.byref(pl8.info), A, A, A, None, A, A,
                              None, 0.07, A, A, A, 1 << 40, None) == 1   # missing scales
    if info.num_combine:
        assert lib.mla_combine(ctypes.byref(shape), ctypes.byref(info), A, None, 1 << 40, None, A,
                               A, None) == 1
        assert lib.mla_combine(ctypes.byref(shape), ctypes.byref(info), A, A, 16, None, A, A,
                               None) == 5


def test_check_validates_before_any_launch(lib):
    shape = _shape(B=2)
    pl = mla.plan(shape, np.array([100, 3000], np.int32), num_workgroups=64, upload=False)
    A = 0x10000   # aligned fake device addresses; never dereferenced on these paths

    def chk(info=pl.info, plan=A, bt=A, kvl=A, ql=None, err=A, sh=shape):
        return lib.mla_decode_check(ctypes.byref(sh), ctypes.byref(info), plan, bt, kvl, ql, err,
                                    None)

    assert chk(plan=None) == 1 and chk(err=None) == 1 and chk(bt=None) == 1
    assert chk(kvl=None) == 1
    assert chk(plan=A + 4) == 4 and chk(err=A + 2) == 4 and chk(ql=A + 1) == 4
    bad = mla.PlanInfo.from_buffer_copy(pl.info)
    bad.phases = 3
    assert chk(info=bad) == 7
    bad = mla.PlanInfo.from_buffer_copy(pl.info)
    bad.plan_bytes = 32
    assert chk(info=bad) == 7
    assert chk(sh=_shape(B=2, P=48)) == 3


def test_empty_batch_is_a_noop(lib):
    shape = _shape(B=0)
    pl = mla.plan(shape, np.zeros(0, np.int32), num_workgroups=8, upload=False)
    assert pl.info.num_items == 0
    assert lib.mla_decode_fwd(ctypes.byref(shape), ctypes.byref(pl.info), None, None, None, None,
                              None, None, None, 1.0, None, None, None, 0, None) == 0


def test_kv_append_validates_before_any_launch(lib):
    A = 0x10000   # aligned fake device addresses; never dereferenced on these paths

    def app(shape, max_new=2, rows=A, nl=None, bt=A, kvl=A, kv=A, sc=None, sk=None):
        return lib.mla_kv_append(ctypes.byref(shape), max_new, rows, nl, bt, kvl, kv, sc, sk, None)

    shape = _shape(B=2)
    assert app(shape, rows=None) == 1
    assert app(shape, bt=None) == 1
    assert app(shape, kvl=None) == 1
    assert app(shape, kv=None) == 1
    assert app(shape, rows=A + 8) == 4
    assert app(shape, kv=A + 4) == 4
    assert app(shape, sk=A + 2) == 4
    assert app(shape, max_new=0) == 2
    assert app(shape, max_new=1 << 30) == 3      # B * max_new rows past 32-bit indexing
    fp8 = _shape(B=2, kvd=mla.KV_FP8_E4M3)
    assert app(fp8) == 1                          # missing scales
    assert app(fp8, sc=A + 2) == 4
    bad = _shape(B=2)
    bad.d_latent = 256
    assert app(bad) == 3
    # an empty batch is a no-op that reads no pointer
    assert app(_shape(B=0), rows=None, bt=None, kvl=None, kv=None) == 0
    # the binding rejects buffers whose sizes do not match the shape
    import torch
    rows = torch.zeros((2, 2, 576), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        mla.kv_append(shape, rows[:1], torch.zeros(2, 16, dtype=torch.int32),
                      torch.zeros(2, dtype=torch.int32), torch.zeros(1, dtype=torch.int16))
    small = _shape(B=2, pages=2, maxp=2)
    kv = torch.zeros((2, 64, 576), dtype=torch.int16)
    bt = torch.zeros((2, 2), dtype=torch.int32)
    with pytest.raises(ValueError, match="kv_lens"):
        mla.kv_append(small, rows, bt, torch.zeros(3, dtype=torch.int32), kv)
    with pytest.raises(ValueError, match="kv_cache"):
        mla.kv_append(small, rows, bt, torch.zeros(2, dtype=torch.int32), kv[:1])
    with pytest.raises(ValueError, match="skipped"):
        mla.kv_append(small, rows, bt, torch.zeros(2, dtype=torch.int32), kv,
                      skipped=torch.zeros(1, dtype=torch.int64))


def _plan_contents(pl):
    """(per-workgroup item lists, combine entries, image counts) of a plan."""
    h = pl.host
    G, N, C, NP = int(h[2]), int(h[3]), int(h[4]), int(h[5])
    ws = h[int(h[8]):int(h[8]) + G + 1]
    items = h[int(h[9]):int(h[9]) + 8 * N].reshape(N, 8)
    per_wg = [items[ws[g]:ws[g + 1]].tolist() for g in range(G)]
    comb = h[int(h[10]):int(h[10]) + 4 * C].reshape(C, 4).tolist()
    return per_wg, comb, (N, C, NP, int(h[11]))


@pytest.mark.parametrize("seed,B,qmax,G,phases", [
    (0, 64, 1, 256, 1), (1, 128, 2, 256, 1), (2, 16, 1, 256, 1), (3, 7, 2, 64, 2),
    (4, 300, 1, 256, 4), (5, 3, 8, 256, 1), (6, 1, 1, 256, 1), (7, 40, 2, 96, 4),
])
def test_fixed_shape_plan_is_the_plan_padded(monkeypatch, seed, B, qmax, G, phases):
    monkeypatch.setenv("MLA_PHASES", str(phases))
    rng = np.random.default_rng(seed)
    kv = rng.integers(1, 5000, size=B, endpoint=True).astype(np.int32)
    ql = rng.integers(0, qmax, size=B, endpoint=True).astype(np.int32)
    kv = np.maximum(kv, ql).astype(np.int32)
    maxp = int((kv.max() + 63) // 64)
    shape = _shape(B=B, qmax=qmax, pages=int(((kv + 63) // 64).sum()) + 1, maxp=maxp)
    a = mla.plan(shape, kv, ql, num_workgroups=G, upload=False)
    f = mla.plan(shape, kv, ql, num_workgroups=G, upload=False, fixed=True)
    wa, ca, na = _plan_contents(a)
    wf, cf, nf = _plan_contents(f)
    P = G // a.info.phases
    assert f.info.num_workgroups == len(wf) == P * a.info.phases
    assert wf[:len(wa)] == wa and all(not w for w in wf[len(wa):])
    assert cf == ca and nf == na
    _check_partition(shape, f, kv, ql)
    # the launch bounds hold for this plan and for every lengths of the shape
    units = B * ((qmax * shape.num_heads + 127) // 128)
    assert f.info.num_combine == units >= na[1]
    assert f.info.num_partials == 2 * f.info.num_workgroups >= na[2]
    assert na[2] <= 2 * (P - 1)
    lib = mla.load_library()
    assert f.info.plan_bytes == lib.mla_plan_bytes_bound(ctypes.byref(shape), G)
    assert f.info.workspace_bytes == lib.mla_workspace_bytes_bound(ctypes.byref(shape), G)


def test_partials_bound_over_many_lengths():
    # the fixed-shape workspace holds 2 * G partials: the planner never needs more
    rng = np.random.default_rng(17)
    for trial in range(300):
        B = int(rng.integers(1, 200))
        G = int(rng.choice([8, 16, 64, 100, 256]))
        qmax = int(rng.integers(1, 9))
        kv = rng.integers(1, int(rng.choice([64, 2000, 40000])), size=B).astype(np.int32)
        ql = rng.integers(0, qmax, size=B, endpoint=True).astype(np.int32)
        kv = np.maximum(kv, ql).astype(np.int32)
        shape = _shape(B=B, qmax=qmax, H=int(rng.choice([16, 128])),
                       pages=int(((kv + 63) // 64).sum()) + 1, maxp=int((kv.max() + 63) // 64))
        pl = mla.plan(shape, kv, ql, num_workgroups=G, upload=False)
        assert pl.info.num_partials <= 2 * (pl.info.num_workgroups - 1), (trial, B, G)


def test_prefill_validates_before_any_launch(lib):
    A = 0x10000   # aligned fake device addresses; never dereferenced on these paths
    P = mla.PrefillShape

    def quant(s, cu=A, q=A, k=A, v=A, qc=A, qs=A, kc=A, ks=A, vc=A, vs=A):
        return lib.mla_prefill_quantize(ctypes.byref(s), cu, q, k, v, qc, qs, kc, ks, vc, vs, None)

    def attn(s, cu=A, qc=A, qs=A, kc=A, ks=A, vc=A, vs=A, scale=0.07, o=A, lse=A):
        return lib.mla_prefill_attn(ctypes.byref(s), cu, qc, qs, kc, ks, vc, vs, scale, o, lse,
                                    None)

    lens = np.array([300, 1, 0, 129], np.int32)
    n = lib.mla_prefill_num_blocks(lens.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), 4)
    assert n == 3 + 1 + 0 + 2
    neg = np.array([5, -1], np.int32)
    assert lib.mla_prefill_num_blocks(neg.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), 2) == -1
    big = np.full(3, 2 ** 31 - 1, np.int32)
    assert lib.mla_prefill_num_blocks(big.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), 3) > 0
    s = P.make(lens, 4)
    assert (s.num_seqs, s.num_tokens, s.num_blocks, s.d_qk, s.d_v) == (4, 430, 6, 192, 128)
    for kw in ("cu", "q", "k", "v", "qc", "qs", "kc", "ks", "vc", "vs"):
        assert quant(s, **{kw: None}) == 1, kw
    for kw in ("cu", "qc", "qs", "kc", "ks", "vc", "vs", "o", "lse"):
        assert attn(s, **{kw: None}) == 1, kw
    for kw in ("q", "k", "v", "qc", "kc", "vc"):
        assert quant(s, **{kw: A + 8}) == 4, kw
    for kw in ("qs", "ks", "vs", "cu"):
        assert quant(s, **{kw: A + 2}) == 4, kw
    for kw in ("qc", "kc", "vc", "o"):
        assert attn(s, **{kw: A + 8}) == 4, kw
    assert attn(s, lse=A + 1) == 4
    assert attn(s, scale=float("nan")) == 2
    assert attn(s, scale=0.0) == 2 and attn(s, scale=-0.1) == 2
    bad = P.make(lens, 4)
    bad.d_qk = 128
    assert quant(bad) == 3 and attn(bad) == 3
    bad = P.make(lens, 0)
    assert quant(bad) == 2
    bad = P.make(lens, 4)
    bad.num_blocks = bad.num_tokens + 1          # more blocks than tokens
    assert quant(bad) == 3
    huge = P(1, 1 << 30, 4, 192, 128, 1)         # T * H past 32-bit indexing
    assert quant(huge) == 3
    # no tokens: a no-op that reads no pointer
    empty = P.make(np.zeros(2, np.int32), 4)
    assert quant(empty, cu=None, q=None, k=None, v=None, qc=None, qs=None, kc=None, ks=None,
                 vc=None, vs=None) == 0
    assert attn(empty, cu=None, qc=None, qs=None, kc=None, ks=None, vc=None, vs=None, o=None,
                lse=None) == 0


def test_plan_log_line():
    # MLA_LOG=1: one stderr line per host plan with its counts and the keys
    # per workgroup (checked against the plan image); unset: nothing
    code = (
        "import numpy as np, mla_paged_decode_absorbed_amd as mla\n"
        "from tests.test_boundary import _shape\n"
        "kv = np.array([5, 4000, 70, 1, 9000], np.int32)\n"
        "pl = mla.plan(_shape(B=5, qmax=1, maxp=200), kv, None, num_workgroups=32, upload=False)\n"
        "it = pl.items()\n"
        "ws = pl.wg_start()\n"
        "G = pl.info.num_workgroups\n"
        "keys = [int(sum(int(i[3]) - int(i[2]) for i in it[ws[g]:ws[g + 1]])) for g in range(G)]\n"
        "print(G, pl.info.num_items, pl.info.num_partials, pl.info.num_combine, max(keys),\n"
        "      '%.1f' % (sum(keys) / G))\n")
    import os
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    for log in ("1", ""):
        env = dict(os.environ, MLA_LOG=log)
        res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                             env=env, cwd=root, timeout=300)
        assert res.returncode == 0, res.stderr[-2000:]
        lines = [l for l in res.stderr.splitlines() if l.startswith("mla: plan")]
        if not log:
            assert not lines
            continue
        G, n_items, n_part, n_comb, most, mean = res.stdout.split()
        assert lines == [f"mla: plan B 5 H 128 q_max 1 page 64 bf16: {G} workgroups, {n_items} "
                         f"items, {n_part} partials, {n_comb} merged blocks, 1 phase(s); keys per "
                         f"workgroup max {most}, mean {mean}"], lines

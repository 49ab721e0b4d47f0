"""Pins of the float64 oracle against things other than itself (CPU only).

Each test names what fixes the expected value: a closed form, an algebraic
identity with an independently written formulation, a library routine, brute
force, or an invariant of softmax attention.  ``test_planted_mistakes`` plants
plausible mistakes in the oracle (on the CPU) and checks that some pin fails.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import mla_ref
from workloads import MLACase, make_case, workload

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


# ------------------------------------------------------------------ codecs

def test_bf16_decode_all_patterns_match_torch():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = oracle.decode_bf16(bits)
    lib = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], lib[~nan])


def test_e4m3_decode_all_codes_match_torch_and_closed_form():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.decode_e4m3(codes)
    lib = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(lib)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], lib[~nan])
    # closed-form anchors of the format
    assert ours[0x7E] == 448.0 and ours[0xFE] == -448.0
    assert ours[0x38] == 1.0 and ours[0xB8] == -1.0
    assert ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6
    assert ours[0x00] == 0.0 and ours[0x80] == 0.0


# ------------------------------------------------------------------ absorption identity

def _absorbed_vs_expanded(case, b, seed=7, d_n=32, d_v=32):
    """Absorbed oracle output projected by W_UV must equal plain per-head
    attention with keys/values expanded through W_UK / W_UV."""
    rng = np.random.default_rng(seed)
    H, d_c, d_r = case.num_heads, case.d_latent, case.d_rope
    w_uk = rng.standard_normal((H, d_c, d_n)) / math.sqrt(d_c)
    w_uv = rng.standard_normal((H, d_c, d_v)) / math.sqrt(d_c)
    q_nope = rng.standard_normal((H, d_n))
    q_rope = rng.standard_normal((H, d_r))
    # absorbed query: latent part W_UK q_nope, rope part unchanged
    q_abs = np.concatenate([np.einsum("hcn,hn->hc", w_uk, q_nope), q_rope], axis=1)
    c2 = MLACase(**{**case.__dict__, "q": q_abs[None, None].repeat(case.batch, 0)})
    O_lat, lse = mla_ref.mla_decode_ref_seq(c2, b)
    O_abs = np.einsum("hc,hcv->hv", O_lat[0], w_uv)
    L = int(case.kv_lens[b])
    K = mla_ref.gather_latent(case.kv, case.block_table[b], L, case.page_size, case.kv_dtype)
    O_ref, lse_ref = oracle.non_absorbed_ref(K[:, :d_c], K[:, d_c:], q_nope, q_rope,
                                             w_uk, w_uv, case.sm_scale)
    return O_abs, lse[0], O_ref, lse_ref


@pytest.mark.parametrize("b", [0, 1])
def test_absorbed_equals_non_absorbed_tiny(b):
    case = workload("tiny_fp32")
    O_abs, lse, O_ref, lse_ref = _absorbed_vs_expanded(case, b)
    rel = np.linalg.norm(O_abs - O_ref) / np.linalg.norm(O_ref)
    assert rel < 1e-12
    assert np.max(np.abs(lse - lse_ref)) < 1e-12


# ------------------------------------------------------------------ closed cases

def _fp32_case(kv_rows, q_rows, page_size=1, sm_scale=1.0, q_len=1, causal=True, perm_seed=3):
    """One sequence stored in fp32 pages placed by a random permutation."""
    kv_rows = np.asarray(kv_rows, np.float32)
    L, D = kv_rows.shape
    n_pages = (L + page_size - 1) // page_size
    num_pages = n_pages + 3
    perm = np.random.default_rng(perm_seed).permutation(num_pages)
    kv = np.full((num_pages, page_size, D), np.nan, np.float32)
    for j in range(L):
        kv[perm[j // page_size], j % page_size] = kv_rows[j]
    bt = np.full((1, n_pages + 2), -1, np.int32)
    bt[0, :n_pages] = perm[:n_pages]
    q = np.asarray(q_rows, np.float32).reshape(1, q_len, -1, D)
    return MLACase(name="closed", batch=1, num_heads=q.shape[2], d_latent=D - 1, d_rope=1,
                   page_size=page_size, kv_dtype="fp32", causal=causal, sm_scale=sm_scale,
                   kv_lens=np.array([L], np.int32), q_lens=np.array([q_len], np.int32),
                   block_table=bt, q=q, kv=kv)


def test_single_visible_key_returns_its_value():
    rng = np.random.default_rng(11)
    kv = rng.standard_normal((1, 9)).astype(np.float32)
    q = rng.standard_normal((4, 9)).astype(np.float32)
    case = _fp32_case(kv, q, sm_scale=0.3)
    O, LSE = oracle.mla_decode_ref(case)
    for h in range(4):
        assert np.array_equal(O[0, 0, h], kv[0, :8].astype(np.float64))
        s0 = 0.3 * float(np.dot(q[h].astype(np.float64), kv[0].astype(np.float64)))
        assert abs(LSE[0, 0, h] - s0) < 1e-12


def test_zero_query_returns_mean_value_and_log_n():
    rng = np.random.default_rng(12)
    n = 37
    kv = rng.standard_normal((n, 9)).astype(np.float32)
    case = _fp32_case(kv, np.zeros((2, 9)), page_size=4)
    O, LSE = oracle.mla_decode_ref(case)
    mean = kv[:, :8].astype(np.float64).mean(axis=0)
    assert np.max(np.abs(O[0, 0] - mean)) < 1e-14
    assert np.max(np.abs(LSE[0, 0] - math.log(n))) < 1e-14


def test_hand_derived_two_key_weights():
    # scores (s0, s1) = (1, 1 + ln 3): weights 1/4, 3/4; LSE = 1 + ln 4
    v0 = np.array([2.0, 1.0, 0.0])
    v1 = np.array([-2.0, 5.0, 4.0])
    ln3 = math.log(3.0)
    kv = np.array([[*v0, 1.0], [*v1, 1.0 + ln3]], np.float64)
    q = np.array([[0.0, 0.0, 0.0, 1.0]])
    case = _fp32_case(kv.astype(np.float32), q.astype(np.float32), page_size=1)
    # fp32 storage rounds 1 + ln 3; use the stored value for the closed form
    s1 = float(np.float32(1.0 + ln3))
    w1 = 1.0 / (1.0 + math.exp(1.0 - s1))
    O, LSE = oracle.mla_decode_ref(case)
    want = (1 - w1) * v0 + w1 * v1
    assert np.max(np.abs(O[0, 0, 0] - want)) < 1e-12
    assert abs(w1 - 0.75) < 1e-7
    assert abs(LSE[0, 0, 0] - (1.0 + math.log(1.0 + math.exp(s1 - 1.0)))) < 1e-12


def test_hand_derived_causal_two_tokens():
    # q_len 2, kv_len 2: token 0 sees key 0 only -> O = v0; token 1 sees both,
    # with equal scores -> O = (v0 + v1) / 2, LSE = s + ln 2
    v0 = np.array([1.0, 3.0, -1.0])
    v1 = np.array([5.0, -1.0, 2.0])
    kv = np.array([[*v0, 2.0], [*v1, 2.0]], np.float32)
    q = np.array([[0, 0, 0, 1.0], [0, 0, 0, 1.0]], np.float32)    # [t, D] with H = 1
    case = _fp32_case(kv, q, q_len=2, page_size=1, sm_scale=0.5)
    O, LSE = oracle.mla_decode_ref(case)
    assert np.array_equal(O[0, 0, 0], v0)
    assert LSE[0, 0, 0] == 1.0
    assert np.max(np.abs(O[0, 1, 0] - (v0 + v1) / 2)) < 1e-15
    assert abs(LSE[0, 1, 0] - (1.0 + math.log(2.0))) < 1e-15


# ------------------------------------------------------------------ causal reduction

def test_causal_q2_rows_equal_q1_calls_with_shorter_cache():
    case = make_case(kv_lens=[40, 77, 2], q_lens=[2, 2, 2], num_heads=4, d_latent=16,
                     d_rope=8, page_size=8, seed=5)
    O, LSE = oracle.mla_decode_ref(case)
    for b in range(case.batch):
        for t in range(2):
            c1 = MLACase(**{**case.__dict__,
                            "kv_lens": case.kv_lens.copy(), "q_lens": np.ones(case.batch, np.int32),
                            "q": case.q[:, t:t + 1].copy()})
            c1.kv_lens[b] = case.kv_lens[b] - 1 + t
            O1, L1 = oracle.mla_decode_ref(c1, seqs=[b])
            assert np.array_equal(O1[b, 0], O[b, t])
            assert np.array_equal(L1[b, 0], LSE[b, t])


def test_q1_non_causal_flag_is_irrelevant():
    case = make_case(kv_lens=[33, 5], num_heads=4, d_latent=16, d_rope=8, page_size=4, seed=6)
    a = oracle.mla_decode_ref(case)
    b = oracle.mla_decode_ref(MLACase(**{**case.__dict__, "causal": False}))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ------------------------------------------------------------------ LSE and combine

def test_lse_bounds_and_normalisation():
    case = make_case(kv_lens=[129, 64], q_lens=[2, 1], num_heads=8, d_latent=32, d_rope=8,
                     page_size=16, seed=8)
    O, LSE = oracle.mla_decode_ref(case)
    ref = oracle.scalar_mla_ref(make_case(kv_lens=[9, 4], q_lens=[2, 1], num_heads=2,
                                          d_latent=4, d_rope=2, page_size=2, seed=8))
    assert ref  # brute force runs
    for b in range(case.batch):
        L = int(case.kv_lens[b])
        K = mla_ref.gather_latent(case.kv, case.block_table[b], L, case.page_size, "bf16")
        for t in range(int(case.q_lens[b])):
            vis = L - int(case.q_lens[b]) + t + 1
            q = oracle.decode_bf16(case.q[b, t])
            s = case.sm_scale * (q @ K[:vis].T)
            mx = s.max(axis=1)
            assert np.all(mx <= LSE[b, t] + 1e-12)
            assert np.all(LSE[b, t] <= mx + math.log(vis) + 1e-12)
            tot = np.exp(s - LSE[b, t][:, None]).sum(axis=1)
            assert np.max(np.abs(tot - 1.0)) < 1e-12


@pytest.mark.parametrize("n_split", [2, 3, 7])
def test_combine_of_random_key_partitions_reproduces_whole(n_split):
    rng = np.random.default_rng(100 + n_split)
    case = make_case(kv_lens=[300], q_lens=[1], num_heads=8, d_latent=32, d_rope=8,
                     page_size=16, seed=9)
    O, LSE = oracle.mla_decode_ref(case)
    L = 300
    K = mla_ref.gather_latent(case.kv, case.block_table[0], L, 16, "bf16")
    q = oracle.decode_bf16(case.q[0, 0])
    cuts = np.sort(rng.choice(np.arange(1, L), size=n_split - 1, replace=False))
    bounds = [0, *cuts.tolist(), L]
    po, pl = [], []
    for a, z in zip(bounds[:-1], bounds[1:]):
        o, l = oracle.attend_rows(q, K[a:z], K[a:z, :32], case.sm_scale)
        po.append(o)
        pl.append(l)
    # an empty partial (stored O is garbage) must not change the result
    po.append(np.full_like(po[0], np.nan))
    pl.append(np.full_like(pl[0], -np.inf))
    Oc, Lc = oracle.combine_ref(np.stack(po), np.stack(pl))
    assert np.max(np.abs(Oc - O[0, 0])) < 1e-13
    assert np.max(np.abs(Lc - LSE[0, 0])) < 1e-13


def test_combine_all_empty_rows():
    Oc, Lc = oracle.combine_ref(np.full((3, 2, 4), np.nan), np.full((3, 2), -np.inf))
    assert np.all(Oc == 0) and np.all(Lc == -np.inf)


# ------------------------------------------------------------------ brute force, layout invariance

@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8_e4m3", "fp32"])
def test_scalar_loops_match_vectorised(kv_dtype):
    case = make_case(kv_lens=[9, 17, 2], q_lens=[2, 1, 2], num_heads=3, d_latent=6, d_rope=2,
                     page_size=4, kv_dtype=kv_dtype, seed=21, sm_scale=0.4)
    O, LSE = oracle.mla_decode_ref(case)
    ref = oracle.scalar_mla_ref(case)
    for (b, t, h), (o, lse) in ref.items():
        assert np.max(np.abs(O[b, t, h] - o)) < 1e-13
        assert abs(LSE[b, t, h] - lse) < 1e-13
    assert len(ref) == 3 * (2 + 1 + 2)
    # padded row (b=1, t=1) is left untouched (NaN)
    assert np.all(np.isnan(O[1, 1]))


def _relayout(case, page_size, perm_seed):
    """Same logical tokens, new page size and a new random page placement."""
    B, D = case.batch, case.d_qk
    rows, scales = [], []
    for b in range(B):
        L = int(case.kv_lens[b])
        n = (L + case.page_size - 1) // case.page_size
        pages = case.block_table[b, :n]
        rows.append(case.kv[pages].reshape(-1, D)[:L])
        if case.kv_scale is not None:
            scales.append(case.kv_scale[pages].reshape(-1)[:L])
    n_pages = [(int(L) + page_size - 1) // page_size for L in case.kv_lens]
    num = sum(n_pages) + 5
    perm = np.random.default_rng(perm_seed).permutation(num)
    kv = np.zeros((num, page_size, D), case.kv.dtype)
    sc = np.zeros((num, page_size), np.float32) if case.kv_scale is not None else None
    bt = np.full((B, max(n_pages)), -1, np.int32)
    off = 0
    for b in range(B):
        for i in range(n_pages[b]):
            bt[b, i] = perm[off + i]
            seg = rows[b][i * page_size:(i + 1) * page_size]
            kv[perm[off + i], :len(seg)] = seg
            if sc is not None:
                sc[perm[off + i], :len(seg)] = scales[b][i * page_size:(i + 1) * page_size]
        off += n_pages[b]
    return MLACase(**{**case.__dict__, "page_size": page_size, "kv": kv, "kv_scale": sc,
                      "block_table": bt})


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8_e4m3"])
def test_page_size_and_permutation_invariance(kv_dtype):
    case = make_case(kv_lens=[130, 64, 1], q_lens=[2, 1, 1], num_heads=4, d_latent=32,
                     d_rope=8, page_size=16, kv_dtype=kv_dtype, seed=31)
    O, LSE = oracle.mla_decode_ref(case)
    for P, s in [(1, 1), (16, 2), (64, 3), (7, 4)]:
        O2, L2 = oracle.mla_decode_ref(_relayout(case, P, s))
        assert np.array_equal(O2, O, equal_nan=True)
        assert np.array_equal(L2, LSE, equal_nan=True)


def test_poisoned_slots_are_never_read():
    case = workload("tiny_fp32")
    O, LSE = oracle.mla_decode_ref(case)
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(LSE))
    # page tails and spare pages really are NaN in the input
    assert np.isnan(case.kv).any()


# ------------------------------------------------------------------ planted mistakes

def _pins_pass():
    """Run a compact set of the pins above; True if all pass."""
    try:
        test_absorbed_equals_non_absorbed_tiny(0)
        test_single_visible_key_returns_its_value()
        test_zero_query_returns_mean_value_and_log_n()
        test_hand_derived_two_key_weights()
        test_hand_derived_causal_two_tokens()
        test_lse_bounds_and_normalisation()
        test_combine_of_random_key_partitions_reproduces_whole(3)
        test_scalar_loops_match_vectorised("bf16")
    except AssertionError:
        return False
    return True


def _mut_attend_drop_rope(q_rows, keys, values, sm_scale):
    d = values.shape[1]
    return ORIG_ATTEND(q_rows[:, :d], keys[:, :d], values, sm_scale)


def _mut_attend_log2(q_rows, keys, values, sm_scale):
    o, lse = ORIG_ATTEND(q_rows, keys, values, sm_scale)
    return o, lse / math.log(2.0)


def _mut_attend_no_scale(q_rows, keys, values, sm_scale):
    return ORIG_ATTEND(q_rows, keys, values, 1.0)


def _mut_attend_values_shifted(q_rows, keys, values, sm_scale):
    d = values.shape[1]
    return ORIG_ATTEND(q_rows, keys, keys[:, keys.shape[1] - d:], sm_scale)


def _mut_attend_unnormalised(q_rows, keys, values, sm_scale):
    o, lse = ORIG_ATTEND(q_rows, keys, values, sm_scale)
    return o * np.exp(lse)[:, None] / np.exp(lse).max(), lse


def _mut_visible_off_by_one(kv_len, q_len, t, causal):
    return int(kv_len - q_len + t) if causal else int(kv_len)


ORIG_ATTEND = mla_ref.attend_rows


@pytest.mark.parametrize("target,mutant", [
    ("attend_rows", _mut_attend_drop_rope),
    ("attend_rows", _mut_attend_log2),
    ("attend_rows", _mut_attend_no_scale),
    ("attend_rows", _mut_attend_values_shifted),
    ("attend_rows", _mut_attend_unnormalised),
    ("visible_keys", _mut_visible_off_by_one),
])
def test_planted_mistakes_are_caught(monkeypatch, target, mutant):
    assert _pins_pass()
    monkeypatch.setattr(mla_ref, target, mutant)
    if target == "attend_rows":
        monkeypatch.setattr(oracle, "attend_rows", mutant)
    assert not _pins_pass()

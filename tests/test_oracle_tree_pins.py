"""Pins of the tree-draft oracle (``oracle/tree_ref.py``) against things other
than itself (CPU only): the causal decode oracle (a lower-triangular tree),
one-token decodes over caches rebuilt without the other drafts (the diagonal
tree), pure-Python loops, and the log-sum-exp split of prefix and drafts.
``test_planted_tree_mistakes_are_caught`` plants plausible mistakes.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import tree_ref
from workloads import MLACase, make_case

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _case(seed=3, q_lens=(4, 3, 1, 4), kv_lens=(70, 9, 40, 4), H=4):
    return make_case(kv_lens=list(kv_lens), q_lens=list(q_lens), seed=seed, num_heads=H,
                     page_size=16, sm_scale=1 / math.sqrt(192), max_q_len=max(q_lens))


def _masks(case, kind):
    B, qmax = case.batch, case.max_q_len
    m = np.zeros((B, qmax), np.uint32)
    for b in range(B):
        for t in range(int(case.q_lens[b])):
            if kind == "causal":
                m[b, t] = (1 << (t + 1)) - 1
            elif kind == "diag":
                m[b, t] = 1 << t
            elif kind == "tree":   # a two-branch tree: 0 <- 1, 0 <- 2 <- 3
                parents = {0: [], 1: [0], 2: [0], 3: [0, 2]}
                m[b, t] = (1 << t) | sum(1 << p for p in parents.get(t, []))
    return m


def _rebuild(case, b, rows_idx):
    """A one-sequence case whose cache holds rows rows_idx of sequence b, in
    order, on fresh pages (raw storage bits copied)."""
    P = case.page_size
    n = len(rows_idx)
    pages = (n + P - 1) // P
    kv = np.zeros((pages + 1,) + case.kv.shape[1:], case.kv.dtype)
    sc = None if case.kv_scale is None else np.zeros((pages + 1, P), np.float32)
    for i, j in enumerate(rows_idx):
        src_page, src_slot = case.block_table[b, j // P], j % P
        kv[i // P, i % P] = case.kv[src_page, src_slot]
        if sc is not None:
            sc[i // P, i % P] = case.kv_scale[src_page, src_slot]
    return kv, sc, np.arange(pages + 1, dtype=np.int32)[None, :]


def check_causal_tree_is_the_causal_decode():
    case = _case()
    Ot, Lt = tree_ref.mla_decode_tree_ref(case, _masks(case, "causal"))
    Oc, Lc = oracle.mla_decode_ref(case)
    ok = True
    for b in range(case.batch):
        q = int(case.q_lens[b])
        ok &= np.allclose(Ot[b, :q], Oc[b, :q], rtol=0, atol=1e-12)
        ok &= np.allclose(Lt[b, :q], Lc[b, :q], rtol=0, atol=1e-12)
    return bool(ok)


def check_diagonal_tree_is_one_token_decodes():
    case = _case(seed=4)
    Ot, Lt = tree_ref.mla_decode_tree_ref(case, _masks(case, "diag"))
    ok = True
    for b in range(case.batch):
        L, q = int(case.kv_lens[b]), int(case.q_lens[b])
        for t in range(q):
            rows = list(range(L - q)) + [L - q + t]
            kv, sc, bt = _rebuild(case, b, rows)
            one = MLACase(name="one", batch=1, num_heads=case.num_heads, d_latent=case.d_latent,
                          d_rope=case.d_rope, page_size=case.page_size, kv_dtype=case.kv_dtype,
                          causal=True, sm_scale=case.sm_scale,
                          kv_lens=np.array([len(rows)], np.int32), q_lens=np.array([1], np.int32),
                          block_table=bt, q=case.q[b:b + 1, t:t + 1], kv=kv, kv_scale=sc)
            O1, L1 = oracle.mla_decode_ref(one)
            ok &= np.allclose(Ot[b, t], O1[0, 0], rtol=0, atol=1e-12)
            ok &= np.allclose(Lt[b, t], L1[0, 0], rtol=0, atol=1e-12)
    return bool(ok)


def check_scalar_loops_on_a_branching_tree():
    case = _case(seed=5, q_lens=(4, 4), kv_lens=(6, 4), H=2)
    mask = _masks(case, "tree")
    Ot, Lt = tree_ref.mla_decode_tree_ref(case, mask)
    q = oracle.decode_bf16(case.q)
    ok = True
    for b in range(case.batch):
        L, qb = int(case.kv_lens[b]), int(case.q_lens[b])
        for t in range(qb):
            for h in range(case.num_heads):
                scores, rows = [], []
                for j in range(L):
                    k = j - (L - qb)
                    if k >= 0 and not (int(mask[b, t]) >> k) & 1:
                        continue
                    page, slot = int(case.block_table[b][j // case.page_size]), j % case.page_size
                    row = oracle.decode_bf16(case.kv[page, slot])
                    scores.append(case.sm_scale * sum(float(q[b, t, h, d]) * float(row[d])
                                                      for d in range(case.d_qk)))
                    rows.append(row)
                mx = max(scores)
                ws = [math.exp(s - mx) for s in scores]
                tot = sum(ws)
                o = sum(w / tot * r[:case.d_latent] for w, r in zip(ws, rows))
                ok &= np.allclose(Ot[b, t, h], o, rtol=0, atol=1e-12)
                ok &= abs(Lt[b, t, h] - (mx + math.log(tot))) <= 1e-12
    return bool(ok)


def check_prefix_and_drafts_merge_to_the_whole():
    # the split the GPU path makes: a non-causal decode over the prefix, the
    # drafts each token sees, and a log-sum-exp merge
    case = _case(seed=6, q_lens=(4, 4, 2), kv_lens=(50, 4, 20), H=3)
    mask = _masks(case, "tree")
    Ot, Lt = tree_ref.mla_decode_tree_ref(case, mask)
    prefix = case.kv_lens - case.q_lens
    pre = MLACase(name="prefix", batch=case.batch, num_heads=case.num_heads,
                  d_latent=case.d_latent, d_rope=case.d_rope, page_size=case.page_size,
                  kv_dtype=case.kv_dtype, causal=False, sm_scale=case.sm_scale,
                  kv_lens=prefix.astype(np.int32), q_lens=case.q_lens, block_table=case.block_table,
                  q=case.q, kv=case.kv, kv_scale=case.kv_scale)
    Op, Lp = oracle.mla_decode_ref(pre)
    ok = True
    for b in range(case.batch):
        L, q = int(case.kv_lens[b]), int(case.q_lens[b])
        K = oracle.gather_latent(case.kv, case.block_table[b], L, case.page_size, case.kv_dtype)
        for t in range(q):
            d = [L - q + k for k in range(q) if (int(mask[b, t]) >> k) & 1]
            Od, Ld = oracle.attend_rows(oracle.decode_bf16(case.q[b, t]), K[d], K[d, :case.d_latent],
                                        case.sm_scale)
            Om, Lm = oracle.combine_ref(np.stack([Op[b, t], Od]), np.stack([Lp[b, t], Ld]))
            ok &= np.allclose(Om, Ot[b, t], rtol=0, atol=1e-12)
            ok &= np.allclose(Lm, Lt[b, t], rtol=0, atol=1e-12)
    return bool(ok)


def check_mask_bits_past_the_drafts_are_ignored():
    case = _case(seed=7)
    m = _masks(case, "tree")
    O1, L1 = tree_ref.mla_decode_tree_ref(case, m)
    O2, L2 = tree_ref.mla_decode_tree_ref(case, m | np.uint32(0xFFFFFF00))
    return bool(np.array_equal(O1, O2, equal_nan=True) and np.array_equal(L1, L2, equal_nan=True))


CHECKS = [check_causal_tree_is_the_causal_decode, check_diagonal_tree_is_one_token_decodes,
          check_scalar_loops_on_a_branching_tree, check_prefix_and_drafts_merge_to_the_whole,
          check_mask_bits_past_the_drafts_are_ignored]


@pytest.mark.parametrize("check", CHECKS, ids=[c.__name__ for c in CHECKS])
def test_tree_pin(check):
    assert check()


def _pins_pass():
    for c in CHECKS:
        try:
            if not c():
                return False
        except Exception:
            return False
    return True


ORIG_VIS = tree_ref.tree_visible_keys


def _mut_prefix_off_by_one(kv_len, q_len, mask_word):
    return ORIG_VIS(kv_len + 1, q_len, mask_word)[:-1] if q_len else ORIG_VIS(kv_len, q_len, mask_word)


def _mut_drafts_from_zero(kv_len, q_len, mask_word):
    prefix = int(kv_len) - int(q_len)
    drafts = [k for k in range(int(q_len)) if (int(mask_word) >> k) & 1]
    return np.array(list(range(max(prefix, 0))) + drafts, dtype=np.int64)


def _mut_all_drafts(kv_len, q_len, mask_word):
    return ORIG_VIS(kv_len, q_len, (1 << int(q_len)) - 1)


def _mut_reversed_bits(kv_len, q_len, mask_word):
    rev = 0
    for k in range(int(q_len)):
        if (int(mask_word) >> k) & 1:
            rev |= 1 << (int(q_len) - 1 - k)
    return ORIG_VIS(kv_len, q_len, rev)


@pytest.mark.parametrize("mutant", [_mut_prefix_off_by_one, _mut_drafts_from_zero,
                                    _mut_all_drafts, _mut_reversed_bits])
def test_planted_tree_mistakes_are_caught(monkeypatch, mutant):
    assert _pins_pass()
    monkeypatch.setattr(tree_ref, "tree_visible_keys", mutant)
    assert not _pins_pass()

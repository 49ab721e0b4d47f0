"""Float64 reference for absorbed-MLA paged decode (test infrastructure only).

The plain definition, computed from exactly the bytes the GPU receives:

1. Sequence b holds kv_len L_b keys.  Its latent rows are the first L_b rows of
   the concatenation of cache pages block_table[b, 0..ceil(L_b/P)-1]; each row
   is d_latent + d_rope wide ([latent | rope]).  The values are the first
   d_latent columns of the same rows (the weight-absorbed reading: the value
   up-projection is folded into the output projection, so values stay latent).
2. Query token t (0 <= t < q_b) sees keys j < vis = L_b - q_b + t + 1 when
   causal (the cache already holds the q_b new tokens), else j < L_b.
3. s_j = sm_scale * <q, k_j>;  O = sum_j softmax(s)_j v_j;
   LSE = log(sum_j exp(s_j))  (natural log).  A row with vis <= 0 gives
   O = 0, LSE = -inf.
4. Merging key-axis splits: LSE = log sum_s exp(LSE_s); O = sum_s exp(LSE_s - LSE) O_s.

Sources: KsanaLLM 0.6.0 page (decode-only weight-absorbed MLA), PaddlePaddle
3.0 inference page (draft tokens verified in one decode pass), FlashAttention-3
in DeepSeek-R1 page, chapter 2 (``softmax_lse`` output; split-K), section 3.1
(per-token KV scale), section 4.1 (block table).

Pins (``tests/test_oracle_pins.py``): the absorbed/non-absorbed identity with
random up-projections; one-key and equal-score closed cases; the causal
reduction q_len 2 -> two q_len 1 calls; the LSE normalisation and bounds;
the combine identity on random key partitions; a pure-Python scalar loop; page
permutation invariance; hand-derived golden cases in ``tests/golden/``.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import logsumexp, softmax

from .codecs import decode_bf16, decode_kv_rows


def visible_keys(kv_len: int, q_len: int, t: int, causal: bool) -> int:
    """Number of keys query token t may attend to (bottom-right causal)."""
    return int(kv_len - q_len + t + 1) if causal else int(kv_len)


def gather_latent(kv, block_table_row, kv_len: int, page_size: int, kv_dtype: str,
                  kv_scale=None) -> np.ndarray:
    """Rows 0..kv_len-1 of one sequence's latent cache, decoded to float64."""
    n_pages = (int(kv_len) + page_size - 1) // page_size
    pages = np.asarray(block_table_row[:n_pages], dtype=np.int64)
    D = kv.shape[-1]
    rows = kv[pages].reshape(n_pages * page_size, D)[:kv_len]
    scale = None
    if kv_scale is not None:
        scale = kv_scale[pages].reshape(n_pages * page_size)[:kv_len]
    return decode_kv_rows(rows, kv_dtype, scale)


def attend_rows(q_rows: np.ndarray, keys: np.ndarray, values: np.ndarray, sm_scale: float):
    """Softmax attention of query rows [R, D] over keys [n, D] / values [n, Dv].

    Returns (O [R, Dv], LSE [R]); n == 0 gives O = 0, LSE = -inf."""
    R = q_rows.shape[0]
    if keys.shape[0] == 0:
        return np.zeros((R, values.shape[1])), np.full(R, -np.inf)
    s = sm_scale * (q_rows @ keys.T)                      # [R, n]
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    l = p.sum(axis=1, keepdims=True)
    o = (p @ values) / l
    lse = (m + np.log(l))[:, 0]
    return o, lse


def _q_f64(q: np.ndarray) -> np.ndarray:
    if q.dtype == np.uint16:
        return decode_bf16(q)
    return np.asarray(q, dtype=np.float64)


def mla_decode_ref_seq(case, b: int):
    """Oracle for one sequence b: (O [q_b, H, Dv], LSE [q_b, H])."""
    L = int(case.kv_lens[b])
    qb = int(case.q_lens[b])
    Dv = case.d_latent
    K = gather_latent(case.kv, case.block_table[b], L, case.page_size, case.kv_dtype,
                      case.kv_scale)
    V = K[:, :Dv]
    O = np.zeros((qb, case.num_heads, Dv))
    LSE = np.zeros((qb, case.num_heads))
    for t in range(qb):
        vis = visible_keys(L, qb, t, case.causal)
        vis = max(vis, 0)
        q_rows = _q_f64(case.q[b, t])                      # [H, D]
        O[t], LSE[t] = attend_rows(q_rows, K[:vis], V[:vis], case.sm_scale)
    return O, LSE


def mla_decode_ref(case, seqs=None):
    """Oracle for a whole call, or for the sequences listed in ``seqs``.

    Returns O [B, q_max, H, Dv] and LSE [B, q_max, H]; rows that are not
    computed (padded rows t >= q_b, or sequences not in ``seqs``) are NaN."""
    B, qmax, H = case.batch, case.max_q_len, case.num_heads
    O = np.full((B, qmax, H, case.d_latent), np.nan)
    LSE = np.full((B, qmax, H), np.nan)
    for b in (range(B) if seqs is None else seqs):
        qb = int(case.q_lens[b])
        if qb == 0:
            continue
        O[b, :qb], LSE[b, :qb] = mla_decode_ref_seq(case, b)
    return O, LSE


def combine_ref(partial_o: np.ndarray, partial_lse: np.ndarray):
    """Merge key-axis partial results.

    partial_o [S, R, Dv] (each normalised over its own keys), partial_lse [S, R].
    Returns (O [R, Dv], LSE [R]); rows whose every partial is empty (-inf)
    give O = 0 and LSE = -inf."""
    po = np.asarray(partial_o, dtype=np.float64)
    pl = np.asarray(partial_lse, dtype=np.float64)
    M = pl.max(axis=0)                                    # [R]
    empty = ~np.isfinite(M)
    Msafe = np.where(empty, 0.0, M)
    w = np.exp(pl - Msafe[None, :])                        # [S, R]; exp(-inf) = 0
    tot = w.sum(axis=0)
    lse = np.where(empty, -np.inf, Msafe + np.log(np.where(empty, 1.0, tot)))
    wn = np.where(empty[None, :], 0.0, w / np.where(empty, 1.0, tot)[None, :])
    o = np.zeros(po.shape[1:])
    for s in range(po.shape[0]):
        # a partial with zero weight (an empty key range) contributes nothing,
        # whatever its stored O holds
        o += np.where(wn[s][:, None] > 0, wn[s][:, None] * po[s], 0.0)
    return o, lse


def non_absorbed_ref(latent: np.ndarray, rope: np.ndarray, q_nope: np.ndarray,
                     q_rope: np.ndarray, w_uk: np.ndarray, w_uv: np.ndarray,
                     sm_scale: float):
    """Standard per-head attention with keys and values expanded per head.

    latent [n, d_c], rope [n, d_r], q_nope [H, d_n], q_rope [H, d_r],
    w_uk [H, d_c, d_n], w_uv [H, d_c, d_v].  Head h uses
    k_j = [latent_j @ w_uk[h] ; rope_j], v_j = latent_j @ w_uv[h],
    q = [q_nope[h] ; q_rope[h]].  Returns (O [H, d_v], LSE [H]).

    Independent of ``attend_rows``: scores are built per head from the expanded
    keys, and softmax / log-sum-exp come from scipy."""
    H = q_nope.shape[0]
    outs, lses = [], []
    for h in range(H):
        k = np.concatenate([latent @ w_uk[h], rope], axis=1)     # [n, d_n + d_r]
        v = latent @ w_uv[h]                                     # [n, d_v]
        q = np.concatenate([q_nope[h], q_rope[h]])
        s = sm_scale * (k @ q)
        outs.append(softmax(s) @ v)
        lses.append(logsumexp(s))
    return np.stack(outs), np.array(lses)


def scalar_mla_ref(case):
    """Pure-Python loops over (b, t, h, j, d) for tiny inputs: brute force with
    per-element address arithmetic through the block table."""
    B, H, P = case.batch, case.num_heads, case.page_size
    D, Dv = case.d_qk, case.d_latent
    qf = _q_f64(case.q)
    out = {}
    for b in range(B):
        L, qb = int(case.kv_lens[b]), int(case.q_lens[b])
        for t in range(qb):
            for h in range(H):
                scores = []
                rows = []
                for j in range(L):
                    # key j is hidden from draft token t when it lies after that
                    # token's own position in the cache (cache position L-qb+t)
                    if case.causal and j > L - qb + t:
                        continue
                    page = int(case.block_table[b][j // P])
                    slot = j % P
                    raw = case.kv[page, slot]
                    sc = None if case.kv_scale is None else case.kv_scale[page, slot]
                    row = decode_kv_rows(raw[None, :], case.kv_dtype,
                                         None if sc is None else np.array([sc]))[0]
                    acc = 0.0
                    for d in range(D):
                        acc += float(qf[b, t, h, d]) * float(row[d])
                    scores.append(case.sm_scale * acc)
                    rows.append(row)
                if not scores:
                    out[(b, t, h)] = (np.zeros(Dv), -math.inf)
                    continue
                mx = max(scores)
                ws = [math.exp(s - mx) for s in scores]
                tot = sum(ws)
                o = [0.0] * Dv
                for w, row in zip(ws, rows):
                    for d in range(Dv):
                        o[d] += w / tot * float(row[d])
                out[(b, t, h)] = (np.array(o), mx + math.log(tot))
    return out

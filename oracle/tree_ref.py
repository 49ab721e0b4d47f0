"""Reference for decode with tree-shaped drafts (test infrastructure only).

Speculative decoding verifies all draft tokens of a sequence in one decode
pass (PaddlePaddle 3.0 inference page, speculative decoding section); with
EAGLE-style drafts (top-k candidates per step, several draft tokens: the
Dewu DeepSeek deployment slides launch SGLang that way) the drafts form a
tree, and a draft token attends to the cached prefix and to the drafts on its
own branch only.

The plain definition, for sequence b with L cached keys of which the last q
are this step's draft tokens (draft k at cache position L - q + k), and a mask
word per draft token t (bit k set: t sees draft k):

  keys visible to t = { j < L - q }  united with  { L - q + k : bit k of mask[b, t] }

and softmax attention over them exactly as for the decode (scores
scale * <q, c_j>, values the latent columns, natural-log LSE).  Bits k >= q
are ignored.  A lower-triangular mask (bit k for k <= t) is the causal decode.

Pins (``tests/test_oracle_tree_pins.py``): the lower-triangular mask equals
the causal decode oracle; the diagonal mask equals, per token, a one-token
decode over a cache without the other drafts; merging a prefix-only
non-causal decode with the draft-only attention by log-sum-exp reproduces
the whole (the split the GPU path uses); and planted mistakes are caught.
"""
from __future__ import annotations

import numpy as np

from .mla_ref import _q_f64, attend_rows, gather_latent


def tree_visible_keys(kv_len: int, q_len: int, mask_word: int) -> np.ndarray:
    """Cache positions visible to a draft token with this mask word."""
    prefix = int(kv_len) - int(q_len)
    drafts = [prefix + k for k in range(int(q_len)) if (int(mask_word) >> k) & 1]
    return np.array(list(range(max(prefix, 0))) + drafts, dtype=np.int64)


def mla_decode_tree_ref_seq(case, tree_mask, b: int):
    """One sequence b: (O [q_b, H, Dv], LSE [q_b, H])."""
    L, qb = int(case.kv_lens[b]), int(case.q_lens[b])
    Dv = case.d_latent
    K = gather_latent(case.kv, case.block_table[b], L, case.page_size, case.kv_dtype,
                      case.kv_scale)
    O = np.zeros((qb, case.num_heads, Dv))
    LSE = np.zeros((qb, case.num_heads))
    for t in range(qb):
        vis = tree_visible_keys(L, qb, int(tree_mask[b][t]))
        O[t], LSE[t] = attend_rows(_q_f64(case.q[b, t]), K[vis], K[vis, :Dv], case.sm_scale)
    return O, LSE


def mla_decode_tree_ref(case, tree_mask, seqs=None):
    """O [B, q_max, H, Dv] and LSE [B, q_max, H] for tree-masked drafts;
    tree_mask [B, q_max] uint32.  Rows not computed are NaN."""
    B, qmax, H, Dv = case.batch, case.max_q_len, case.num_heads, case.d_latent
    O = np.full((B, qmax, H, Dv), np.nan)
    LSE = np.full((B, qmax, H), np.nan)
    mask = np.asarray(tree_mask, dtype=np.uint32)
    for b in (range(B) if seqs is None else seqs):
        qb = int(case.q_lens[b])
        if qb == 0:
            continue
        O[b, :qb], LSE[b, :qb] = mla_decode_tree_ref_seq(case, mask, b)
    return O, LSE

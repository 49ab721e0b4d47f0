"""Float64 CPU oracle for absorbed-MLA decode over a paged latent cache.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
path (no kernels, headers, helpers, tables or constants) and decodes the raw
storage bits itself.

What it computes, and where the pages state it:

* Weight-absorbed MLA decode: every query head carries one vector scored
  directly against the shared compressed (latent) cache, with the up-projection
  folded into the query and into the output projection, so the per-head values
  are the latent rows themselves (KsanaLLM 0.6.0 page, the prefill/decode
  disaggregation section on the decode-only weight-absorbed MLA path).
* Softmax attention whose normaliser is also returned as a natural-log
  log-sum-exp (FlashAttention-3-in-DeepSeek-R1 page, chapter 2, the kernel
  signature carrying ``softmax_lse``).
* More than one query token per sequence in the decode step, all draft tokens
  verified in one pass at the original batch size (PaddlePaddle 3.0 inference
  page, speculative-decoding section on draft-token verification).  The causal
  reading: query token t of q_len sees keys j <= kv_len - q_len + t.
* Splitting the key axis and merging partial results by their log-sum-exp
  (FlashAttention-3 page, chapter 2, "split-K").
* Paged cache addressed through a block table (FlashAttention-3 page, section
  4.1 on the PagedAttention block table; Dewu deployment slides on
  PagedAttention).
* fp8-e4m3 cache with one scale per cached token, symmetric, zero-point 0
  (FlashAttention-3 page, section 3.1, per-token KV calibration; PaddlePaddle
  3.0 page on low-bit KV cache).
* Writing a step's new tokens into their page slots, quantizing them with
  that per-token scale for an e4m3 cache (``append_ref``).
* Tree-shaped drafts: each draft token sees the cached prefix and the drafts
  its mask names (``tree_ref``; EAGLE-style drafts of the Dewu deployment
  slides, verified in one pass as on the PaddlePaddle 3.0 page).
* SageAttention-style quantized causal prefill: INT8 Q and K, FP8 V and P,
  blocked online softmax (``prefill_ref``; PaddlePaddle 3.0 page, the
  long-sequence SageAttention paragraph).

Every function below is pinned by ``tests/test_oracle_pins.py`` (the
append by ``tests/test_oracle_append_pins.py``, the tree drafts by
``tests/test_oracle_tree_pins.py``, the prefill by
``tests/test_oracle_prefill_pins.py``) against something other than
itself (closed forms, the non-absorbed identity, brute force, library casts,
invariants); see each docstring.
"""
from .codecs import decode_bf16, decode_e4m3, decode_kv_rows  # noqa: F401
from .mla_ref import (  # noqa: F401
    attend_rows,
    gather_latent,
    mla_decode_ref,
    mla_decode_ref_seq,
    combine_ref,
    non_absorbed_ref,
    scalar_mla_ref,
    visible_keys,
)
from .append_ref import (  # noqa: F401
    append_positions,
    encode_e4m3,
    kv_append_ref,
    quantize_rows_e4m3,
)
from .tree_ref import mla_decode_tree_ref, mla_decode_tree_ref_seq, tree_visible_keys  # noqa: F401
from .prefill_ref import (  # noqa: F401
    quantize_case, quantize_p, quantize_rows_int8, quantize_v_blocks, sage_prefill_ref,
)

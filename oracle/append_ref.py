"""Reference for the cache append (test infrastructure only).

The plain definition:

1. Placement.  Token t (0 <= t < n_b) of the n_b new tokens of sequence b is
   cache position p = kv_len_b - n_b + t (the cache length already counts the
   new tokens, as for the decode).  Position p is slot p mod P of page
   block_table[b, p div P] (FlashAttention-3 in DeepSeek-R1 page, section 4.1,
   the PagedAttention block table).  A token whose position lies outside
   [0, max_pages * P), whose page id lies outside the pool, or whose sequence
   claims more than max_new new tokens is not written and is counted as
   skipped.  Nothing else in the cache changes.
2. bf16 cache: the row's bits are stored unchanged.
3. e4m3 cache: one symmetric scale per token (FlashAttention-3 page, section
   3.1: the row's largest magnitude over the largest code magnitude, zero
   point 0; its int8 range 127 becomes e4m3's 448 here, the 8-bit KV cache of
   the PaddlePaddle 3.0 inference page).  In fp32: s = max|x| / 448, s = 1 for
   an all-zero row; y = x / s clamped to [-448, 448]; the stored code is the
   e4m3 value nearest to y, ties going to the code with an even mantissa.
   The scale and the quotient are computed in fp32 because they decide
   integer codes: this is the precision the kernel takes them in.

Pins (``tests/test_oracle_append_pins.py``): the encoder maps every finite code's
value back to that code, sends every midpoint between neighbouring codes to
the even one, and agrees with the library cast ``torch.float8_e4m3fn`` on
random fp32 values over the whole range; the largest element of each row gets
code +-448; the round trip stays within half a code step; placement is checked
against a pure-Python loop and, through the decode oracle's own gather, reads
back the appended rows at positions kv_len - n .. kv_len - 1.
"""
from __future__ import annotations

import numpy as np

from .codecs import decode_e4m3

E4M3_MAX = 448.0


def _nonneg_e4m3_table():
    """(values, codes): the 127 non-negative finite e4m3 values, ascending."""
    codes = np.arange(0x00, 0x7F, dtype=np.uint8)          # 0x7F is NaN
    vals = decode_e4m3(codes)
    order = np.argsort(vals, kind="stable")
    return vals[order], codes[order]


_TABLE = _nonneg_e4m3_table()


def encode_e4m3(y) -> np.ndarray:
    """Nearest e4m3 code to each value of ``y`` (|y| <= 448), ties to the
    even code; the sign is kept (-0.0 -> 0x80)."""
    y = np.asarray(y, dtype=np.float64)
    if np.any(~np.isfinite(y)) or np.any(np.abs(y) > E4M3_MAX):
        raise ValueError("encode_e4m3 takes finite values within +-448")
    vals, codes = _TABLE
    a = np.abs(y)
    hi = np.clip(np.searchsorted(vals, a, side="left"), 0, len(vals) - 1)
    lo = np.clip(hi - 1, 0, len(vals) - 1)
    d_lo, d_hi = a - vals[lo], vals[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((codes[hi] & 1) == 0))
    mag = np.where(pick_hi, codes[hi], codes[lo]).astype(np.uint8)
    neg = np.signbit(y)
    return np.where(neg, mag | np.uint8(0x80), mag).astype(np.uint8)


def quantize_rows_e4m3(x_f32):
    """Rows [..., D] of fp32 values -> (codes [..., D] uint8, scale [...] fp32)."""
    x = np.asarray(x_f32, dtype=np.float32)
    amax = np.max(np.abs(x), axis=-1)
    scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    scale = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    y = (x / scale[..., None]).astype(np.float32)
    y = np.clip(y, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
    return encode_e4m3(y), scale


def append_positions(kv_lens, new_lens, max_new: int, block_table, page_size: int,
                     num_pages: int):
    """[(b, t, page, slot)] of every token that is written, and the number of
    skipped tokens."""
    out, skipped = [], 0
    B = len(kv_lens)
    max_pages = block_table.shape[1]
    for b in range(B):
        n = int(new_lens[b]) if new_lens is not None else int(max_new)
        for t in range(min(max(n, 0), max_new)):
            p = int(kv_lens[b]) - n + t
            if n > max_new or p < 0 or p >= max_pages * page_size:
                skipped += 1
                continue
            page = int(block_table[b, p // page_size])
            if page < 0 or page >= num_pages:
                skipped += 1
                continue
            out.append((b, t, page, p % page_size))
    return out, skipped


def kv_append_ref(kv, kv_scale, block_table, kv_lens, new_lens, new_rows_bits, page_size: int,
                  kv_dtype: str):
    """Returns (kv', kv_scale', skipped) after writing the new tokens.

    kv [pages, P, D] uint16 bf16 bits or uint8 e4m3 codes; kv_scale [pages, P]
    fp32 (e4m3) or None; new_rows_bits [B, max_new, D] uint16 bf16 bits."""
    kv = np.array(kv, copy=True)
    kv_scale = None if kv_scale is None else np.array(kv_scale, dtype=np.float32, copy=True)
    max_new = new_rows_bits.shape[1]
    writes, skipped = append_positions(kv_lens, new_lens, max_new, np.asarray(block_table),
                                       page_size, kv.shape[0])
    for b, t, page, slot in writes:
        row = np.asarray(new_rows_bits[b, t], dtype=np.uint16)
        if kv_dtype == "bf16":
            kv[page, slot] = row
        elif kv_dtype == "fp8_e4m3":
            x = (row.astype(np.uint32) << np.uint32(16)).view(np.float32)
            codes, s = quantize_rows_e4m3(x)
            kv[page, slot] = codes
            kv_scale[page, slot] = s
        else:
            raise ValueError(kv_dtype)
    return kv, kv_scale, skipped

"""Reference for SageAttention-style quantized prefill (test infrastructure only).

The PaddlePaddle 3.0 inference page (long-sequence inference, the
SageAttention paragraph) describes a prefill attention for DeepSeek's head
dim 192 whose data types change by stage: Q and K are quantized to INT8 on
the fly and V to FP8; the INT32 products Q*K^T are converted to FP32 and
dequantized; an online softmax runs over them; its probabilities P are
quantized to FP8 and multiplied with the FP8 V, and V's quantization is
undone afterwards to give O.

Readings (the page fixes no granularity, scale rule or block size):

* Q: one symmetric scale per (token, head) row, scale = max|x| / 127 in fp32
  (1 for an all-zero row); code = x / scale (correctly rounded fp32
  quotient) rounded to nearest, ties to even, clamped to +-127.
* K: the same rule with one scale per (128-token block of a sequence, head),
  the maximum taken over the block's tokens and all 192 dims: a block's
  scores then share one key scale.
* V: one power-of-two scale per (128-token block, head, channel), the
  smallest 2^e with max|v| / 2^e <= 448 over the block's tokens (e >= -127;
  2^0 for an all-zero channel); code = the e4m3 code nearest to v / 2^e, an
  exact quotient.  V's quantization is undone after each block's P V
  product, which is where a per-channel scale can come off; a power of two
  is what a block-scaled (e8m0) matrix instruction applies by itself.
* The online softmax steps over the keys in blocks of 128 from the start of
  the sequence: per block the running max is raised, P = exp(s - m) for the
  block's visible keys, l and the accumulator are rescaled by exp(m_old -
  m_new); P enters the product as e4m3(448 P) / 448 (448 maps P's range
  [0, 1] onto e4m3's), while l sums the unquantized P.
* Scores s = (q_codes . k_codes) * q_scale * k_scale * sm_scale; causal
  within a sequence (token i sees keys j <= i); LSE = m + ln l (natural log).
* Shapes: per head, Q and K 192 wide (128 + 64 rope), V 128 wide; sequences
  packed along the token axis by cu_seqlens.

With every quantizer replaced by the identity the blocked recurrence is
plain softmax attention; ``tests/test_oracle_prefill_pins.py`` checks that
against the decode oracle's attention, closed forms (a sequence's first token
returns its own dequantized V row; zero queries give the mean of the visible
dequantized V rows and LSE ln n), brute-force nearest codes, an error bound
against unquantized attention, and planted mistakes.
"""
from __future__ import annotations

import numpy as np

from .append_ref import encode_e4m3
from .codecs import decode_bf16, decode_e4m3

KEY_BLOCK = 128
P_SCALE = 448.0
INT8_MAX = 127
E4M3_MAX = 448.0


def _f32(x_bits_or_values) -> np.ndarray:
    x = np.asarray(x_bits_or_values)
    if x.dtype == np.uint16:
        return decode_bf16(x).astype(np.float32)
    return x.astype(np.float32)


def quantize_rows_int8(x):
    """Rows [..., D] (bf16 bits or fp32) -> (codes int8 [..., D], scale fp32 [...])."""
    x = _f32(x)
    amax = np.max(np.abs(x), axis=-1)
    scale = (amax / np.float32(INT8_MAX)).astype(np.float32)
    scale = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    y = (x / scale[..., None]).astype(np.float32)          # correctly rounded fp32
    codes = np.clip(np.rint(y), -INT8_MAX, INT8_MAX)       # rint: ties to even
    return codes.astype(np.int8), scale


def num_blocks(seqlens) -> int:
    return int(sum((int(n) + KEY_BLOCK - 1) // KEY_BLOCK for n in seqlens))


def _blocks(cu_seqlens):
    """(t0, t1) of every 128-token block, sequences in order."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    return [(t0, min(t0 + KEY_BLOCK, int(cu[s + 1])))
            for s in range(len(cu) - 1) for t0 in range(int(cu[s]), int(cu[s + 1]), KEY_BLOCK)]


def quantize_k_blocks(k, cu_seqlens):
    """K [T, H, D] (bf16 bits or fp32) -> (codes int8 [T, H, D], scales fp32
    [blocks, H]): one scale per 128-token block and head."""
    x = _f32(k)
    T, H, D = x.shape
    blocks = _blocks(cu_seqlens)
    codes = np.zeros((T, H, D), np.int8)
    scales = np.ones((len(blocks), H), np.float32)
    for bi, (t0, t1) in enumerate(blocks):
        xb = x[t0:t1]                                       # [n, H, D]
        amax = np.max(np.abs(xb), axis=(0, 2))
        sc = (amax / np.float32(INT8_MAX)).astype(np.float32)
        sc = np.where(sc > 0, sc, np.float32(1.0)).astype(np.float32)
        y = (xb / sc[None, :, None]).astype(np.float32)
        codes[t0:t1] = np.clip(np.rint(y), -INT8_MAX, INT8_MAX).astype(np.int8)
        scales[bi] = sc
    return codes, scales


def pow2_scale_exponent(amax) -> np.ndarray:
    """Smallest e >= -127 with amax / 2^e <= 448 (0 where amax is 0), exactly:
    amax = m 2^E with m in [0.5, 1) fits 448 = 0.875 * 2^9 at e = E - 9 when
    m <= 0.875, else at E - 8."""
    a = np.asarray(amax, dtype=np.float64)
    m, E = np.frexp(a)
    e = np.where(m <= 0.875, E - 9, E - 8)
    e = np.maximum(e, -127)
    return np.where(a > 0, e, 0).astype(np.int32)


def quantize_v_blocks(v, cu_seqlens):
    """V [T, H, Dv] (bf16 bits or fp32) -> (codes uint8 [T, H, Dv], scales fp32
    [blocks, H, Dv], powers of two); block index = the sequence's first block
    + key block."""
    x = _f32(v)
    T, H, Dv = x.shape
    blocks = _blocks(cu_seqlens)
    codes = np.zeros((T, H, Dv), np.uint8)
    scales = np.ones((len(blocks), H, Dv), np.float32)
    for bi, (t0, t1) in enumerate(blocks):
        xb = x[t0:t1].astype(np.float64)                    # [n, H, Dv]
        e = pow2_scale_exponent(np.max(np.abs(xb), axis=0))
        y = np.clip(np.ldexp(xb, -e[None]), -E4M3_MAX, E4M3_MAX)   # exact
        codes[t0:t1] = encode_e4m3(y)
        scales[bi] = np.ldexp(np.float32(1.0), e).astype(np.float32)
    return codes, scales


def quantize_p(p) -> np.ndarray:
    """P in [0, 1] as it enters the PV product: e4m3(448 P) / 448."""
    return decode_e4m3(encode_e4m3(np.asarray(p, np.float64) * P_SCALE)) / P_SCALE


def blocked_attend_row(s, values, quant_p: bool = True, block: int = KEY_BLOCK):
    """One query row: scores s [n] over its visible keys (in key order from
    the sequence start) and their values [n, Dv] -> (O [Dv], LSE), by the
    blocked online softmax."""
    n = s.shape[0]
    if n == 0:
        return np.zeros(values.shape[1]), -np.inf
    m, l = -np.inf, 0.0
    acc = np.zeros(values.shape[1])
    for b0 in range(0, n, block):
        sb = s[b0:b0 + block]
        m_new = max(m, float(sb.max()))
        alpha = np.exp(m - m_new)                            # 0 on the first block
        p = np.exp(sb - m_new)
        l = l * alpha + float(p.sum())
        pu = quantize_p(p) if quant_p else p
        acc = acc * alpha + pu @ values[b0:b0 + block]
        m = m_new
    return acc / l, m + np.log(l)


def quantize_case(case):
    """The three quantizers applied to a prefill case's bf16 inputs."""
    qc, qs = quantize_rows_int8(case.q)
    kc, ks = quantize_k_blocks(case.k, case.cu_seqlens)
    vc, vs = quantize_v_blocks(case.v, case.cu_seqlens)
    return qc, qs, kc, ks, vc, vs


def sage_prefill_ref(case, rows=None, quantized=None):
    """O [T, H, Dv] and LSE [T, H] of the quantized causal prefill (float64).
    ``rows``: iterable of (token, head) to compute (default: all); others are
    NaN.  ``quantized``: the output of ``quantize_case`` if already at hand."""
    qc, qs, kc, ks, vc, vs = quantize_case(case) if quantized is None else quantized
    T, H = case.num_tokens, case.num_heads
    Dv = case.d_v
    cu = np.asarray(case.cu_seqlens, dtype=np.int64)
    O = np.full((T, H, Dv), np.nan)
    LSE = np.full((T, H), np.nan)
    if rows is None:
        rows = [(t, h) for t in range(T) for h in range(H)]
    seq_of = np.searchsorted(cu, np.arange(T), side="right") - 1
    blk0 = np.concatenate([[0], np.cumsum((np.diff(cu) + KEY_BLOCK - 1) // KEY_BLOCK)])
    vdq_cache = {}
    for t, h in rows:
        s = int(seq_of[t])
        t0 = int(cu[s])
        i = t - t0
        key = (s, h)
        if key not in vdq_cache:
            n_s = int(cu[s + 1]) - t0
            vals = decode_e4m3(vc[t0:t0 + n_s, h]).astype(np.float64)
            for kb in range((n_s + KEY_BLOCK - 1) // KEY_BLOCK):
                vals[kb * KEY_BLOCK:(kb + 1) * KEY_BLOCK] *= vs[int(blk0[s]) + kb, h]
            vdq_cache = {key: vals}
        vals = vdq_cache[key]
        ints = kc[t0:t + 1, h].astype(np.int64) @ qc[t, h].astype(np.int64)      # exact
        kscale = np.repeat(ks[int(blk0[s]):int(blk0[s + 1]), h].astype(np.float64),
                           KEY_BLOCK)[:i + 1]
        sc = ints.astype(np.float64) * float(qs[t, h]) * kscale
        sc = sc * case.sm_scale
        O[t, h], LSE[t, h] = blocked_attend_row(sc, vals[:i + 1])
    return O, LSE

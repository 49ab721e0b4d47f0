"""Helpers shared by the prefill parity tests (emulated and GPU): the V-code
layout of mla_prefill_quantize undone, and comparisons with the oracle."""
import math

import numpy as np

from oracle import decode_bf16, prefill_ref

# O / LSE bars of the quantized path (the e4m3 bar of the decode)
O_MAX_ABS, O_REL_L2, LSE_TOL = 6e-2, 2e-2, 1e-3


def key_positions():
    """pos[k] = byte of key k (0..127) in a (block, head, channel) row:
    key 16 a + 4 g + r sits at byte 32 g + 4 a + r."""
    k = np.arange(128)
    a, g, r = k >> 4, (k >> 2) & 3, k & 3
    return 32 * g + 4 * a + r


def natural_v_codes(vt, cu_seqlens, T):
    """[blocks, H, 128 ch, 128 pos] -> ([T, H, 128] codes, padding bytes all zero?)"""
    pos = key_positions()
    nb, H = vt.shape[:2]
    out = np.zeros((T, H, 128), np.uint8)
    pad_zero = True
    blk = 0
    cu = np.asarray(cu_seqlens)
    for s in range(len(cu) - 1):
        for t0 in range(int(cu[s]), int(cu[s + 1]), 128):
            n = min(128, int(cu[s + 1]) - t0)
            rows = vt[blk][:, :, pos]                 # [H, ch, key]
            out[t0:t0 + n] = np.transpose(rows[:, :, :n], (2, 0, 1))
            pad_zero &= bool(np.all(rows[:, :, n:] == 0))
            blk += 1
    assert blk == nb
    return out, pad_zero


def check_quantized(case, got):
    qc, qs, kc, ks, vc, vs = prefill_ref.quantize_case(case)
    assert np.array_equal(got["qc"], qc)
    assert np.array_equal(got["qs"].view(np.uint32), qs.view(np.uint32))
    assert np.array_equal(got["kc"], kc)
    assert np.array_equal(got["ks"].view(np.uint32), ks.view(np.uint32))
    nat, pad_zero = natural_v_codes(got["vc"], case.cu_seqlens, case.num_tokens)
    assert np.array_equal(nat, vc)
    assert pad_zero
    assert np.array_equal(got["vs"].view(np.uint32), vs.view(np.uint32))
    return qc, qs, kc, ks, vc, vs


def check_attention(case, o_bits, lse, rows=None, quantized=None):
    """O (bf16 bits) and LSE against the oracle on ``rows`` [(t, h)] (all by
    default); returns (max abs, rel-L2, max LSE error)."""
    O, L = prefill_ref.sage_prefill_ref(case, rows=rows, quantized=quantized)
    o = decode_bf16(np.asarray(o_bits)).astype(np.float64)
    sel = ~np.isnan(L)
    d = o[sel] - O[sel]
    assert np.all(np.isfinite(o[sel]))
    worst = float(np.abs(d).max()) if d.size else 0.0
    rel = math.sqrt(float((d ** 2).sum()) / max(float((O[sel] ** 2).sum()), 1e-300))
    dl = float(np.abs(np.asarray(lse, np.float64)[sel] - L[sel]).max()) if d.size else 0.0
    assert worst <= O_MAX_ABS, worst
    assert rel <= O_REL_L2, rel
    assert dl <= LSE_TOL, dl
    return worst, rel, dl

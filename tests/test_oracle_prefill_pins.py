"""Pins of the quantized-prefill oracle (``oracle/prefill_ref.py``) against
things other than itself (CPU only):

* the blocked online softmax with P unquantized equals the decode oracle's
  plain softmax attention, for any block size;
* inputs built to quantize exactly (Q rows, and K blocks of 128 tokens, =
  integer codes times a power of two with a +-127 element; V = e4m3 values
  times a power of two with +-448 in every block and channel) make the whole
  pipeline plain causal attention up to P's rounding, whose effect is bounded
  by e4m3's relative step;
* closed forms: a sequence's first token returns its own dequantized V row
  and LSE = its one score; zero query rows give the mean of the visible V
  rows and LSE = ln n;
* brute-force nearest codes for all three quantizers, hand-made ties;
* planted mistakes are caught.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import prefill_ref
from workloads.prefill import PrefillCase, make_prefill_case, _bf16_bits

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

E4M3_VALUES = oracle.decode_e4m3(np.arange(256, dtype=np.uint8))
FINITE = np.isfinite(E4M3_VALUES)


def _exact_case(seqlens, H=2, seed=0, zero_q_rows=()):
    """Inputs whose quantization is exact (see the module docstring)."""
    rng = np.random.default_rng(seed)
    cu = np.concatenate([[0], np.cumsum(seqlens)]).astype(np.int32)
    T = int(cu[-1])

    def int_rows(shape):
        c = rng.integers(-126, 127, size=shape).astype(np.float32)
        idx = rng.integers(0, shape[-1], size=shape[:-1])
        sign = rng.choice([-1.0, 1.0], size=shape[:-1])
        np.put_along_axis(c, idx[..., None], (127.0 * sign)[..., None].astype(np.float32), -1)
        p2 = np.exp2(rng.integers(-6, 3, size=shape[:-1])).astype(np.float32)
        return c * p2[..., None]

    q = int_rows((T, H, 192))
    for t in zero_q_rows:
        q[t] = 0.0
    # K: one power of two and one +-127 per (128-token block, head)
    k = rng.integers(-126, 127, size=(T, H, 192)).astype(np.float32)
    for s in range(len(seqlens)):
        for t0 in range(int(cu[s]), int(cu[s + 1]), 128):
            t1 = min(t0 + 128, int(cu[s + 1]))
            for h in range(H):
                k[int(rng.integers(t0, t1)), h, int(rng.integers(0, 192))] = 127.0 * rng.choice([-1, 1])
                k[t0:t1, h] *= np.float32(2.0 ** int(rng.integers(-6, 3)))
    pos = E4M3_VALUES[FINITE & (np.abs(E4M3_VALUES) < 448)]
    v = rng.choice(pos, size=(T, H, 128)).astype(np.float32)
    for s in range(len(seqlens)):
        for t0 in range(int(cu[s]), int(cu[s + 1]), 128):
            t1 = min(t0 + 128, int(cu[s + 1]))
            for h in range(H):
                # +-448 somewhere in every channel of the block, times 2^b
                rows = rng.integers(t0, t1, size=128)
                v[rows, h, np.arange(128)] = 448.0 * rng.choice([-1.0, 1.0], size=128)
                v[t0:t1, h] *= np.float32(2.0 ** int(rng.integers(-8, 2)))
    case = PrefillCase(name="exact", seqlens=np.asarray(seqlens, np.int32), cu_seqlens=cu,
                       num_heads=H, sm_scale=1 / math.sqrt(192),
                       q=_bf16_bits(q), k=_bf16_bits(k), v=_bf16_bits(v))
    return case, q.astype(np.float64), k.astype(np.float64), v.astype(np.float64)


def check_exact_inputs_quantize_exactly():
    case, q, k, v = _exact_case([200, 7], seed=1)
    qc, qs, kc, ks, vc, vs = prefill_ref.quantize_case(case)
    ok = np.array_equal(qc * qs[..., None].astype(np.float64), q)
    vdq = oracle.decode_e4m3(vc).astype(np.float64)
    blk = 0
    for s in range(case.num_seqs):
        for t0 in range(int(case.cu_seqlens[s]), int(case.cu_seqlens[s + 1]), 128):
            t1 = min(t0 + 128, int(case.cu_seqlens[s + 1]))
            ok &= np.array_equal(kc[t0:t1] * ks[blk][None, :, None].astype(np.float64), k[t0:t1])
            ok &= np.array_equal(vdq[t0:t1] * vs[blk][None], v[t0:t1])
            blk += 1
    return bool(ok) and blk == vs.shape[0]


def check_blocked_softmax_is_plain_softmax():
    rng = np.random.default_rng(2)
    ok = True
    for n in (1, 5, 127, 128, 129, 1000):
        s = rng.standard_normal(n) * 4 + np.linspace(0, 6, n)     # a rising max
        vals = rng.standard_normal((n, 16))
        o_ref, l_ref = oracle.attend_rows(s[None], np.eye(n), vals, 1.0)
        for block in (1, 7, 128, 4096):
            o, l = prefill_ref.blocked_attend_row(s, vals, quant_p=False, block=block)
            ok &= np.allclose(o, o_ref[0], rtol=0, atol=1e-12)
            ok &= abs(l - l_ref[0]) <= 1e-12
    return bool(ok)


def check_pipeline_is_causal_attention_up_to_p_rounding():
    case, q, k, v = _exact_case([300, 1, 130], H=2, seed=3)
    O, L = prefill_ref.sage_prefill_ref(case)
    ok = True
    step = 2.0 ** -4                       # e4m3 relative half step (normal range)
    sub = 2.0 ** -10 / 448.0               # absolute half step below the normal range, in P units
    for s in range(case.num_seqs):
        t0, t1 = int(case.cu_seqlens[s]), int(case.cu_seqlens[s + 1])
        for t in range(t0, t1):
            for h in range(case.num_heads):
                keys, vals = k[t0:t + 1, h], v[t0:t + 1, h]
                o, lse = oracle.attend_rows(q[t, h][None], keys, vals, case.sm_scale)
                sc = case.sm_scale * keys @ q[t, h]
                p = np.exp(sc - sc.max())
                bound = (step * (p @ np.abs(vals)) + sub * np.abs(vals).sum(0)) / p.sum()
                ok &= bool(np.all(np.abs(O[t, h] - o[0]) <= bound * (1 + 1e-9) + 1e-12))
                ok &= abs(L[t, h] - lse[0]) <= 1e-9
    return bool(ok)


def check_first_token_and_zero_query_closed_forms():
    case = make_prefill_case(seqlens=[260, 3, 129], num_heads=2, seed=4)
    zero = [1, 150, 259, 261, 262 + 128]
    for t in zero:
        case.q[t] = 0
    qc, qs, kc, ks, vc, vs = prefill_ref.quantize_case(case)
    O, L = prefill_ref.sage_prefill_ref(case)
    vdq = oracle.decode_e4m3(vc).astype(np.float64)
    ok = True
    blk0 = [0, 3, 4]
    for s in range(case.num_seqs):
        t0, t1 = int(case.cu_seqlens[s]), int(case.cu_seqlens[s + 1])
        for h in range(case.num_heads):
            ok &= np.array_equal(O[t0, h], vdq[t0, h] * vs[blk0[s], h])
            s00 = float(int(qc[t0, h].astype(np.int64) @ kc[t0, h].astype(np.int64)))
            ok &= abs(L[t0, h] - s00 * float(qs[t0, h]) * float(ks[blk0[s], h]) * case.sm_scale) <= 1e-12
        for t in zero:
            if not t0 <= t < t1:
                continue
            n = t - t0 + 1
            for h in range(case.num_heads):
                rows = np.array([vdq[j, h] * vs[blk0[s] + (j - t0) // 128, h] for j in range(t0, t + 1)])
                ok &= np.allclose(O[t, h], rows.mean(0), rtol=0, atol=1e-12)
                ok &= abs(L[t, h] - math.log(n)) <= 1e-12
    return bool(ok)


def check_int8_codes_are_nearest_brute_force():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((40, 192)) * np.exp(rng.uniform(-8, 8, (40, 1)))).astype(np.float32)
    x = oracle.decode_bf16(_bf16_bits(x)).astype(np.float32)
    x[3] = 0.0
    codes, scale = prefill_ref.quantize_rows_int8(_bf16_bits(x))
    ok = True
    cand = np.arange(-127, 128)
    for r in range(x.shape[0]):
        amax = np.float32(np.abs(x[r]).max())
        want_scale = np.float32(amax / np.float32(127)) if amax > 0 else np.float32(1)
        ok &= scale[r] == want_scale
        y = (x[r] / want_scale).astype(np.float32).astype(np.float64)
        d = np.abs(y[:, None] - cand[None, :])
        best = d.min(1, keepdims=True)
        for i in range(192):
            ties = cand[d[i] == best[i, 0]]
            want = ties[0] if len(ties) == 1 else ties[ties % 2 == 0][0]
            ok &= int(codes[r, i]) == int(want)
        if amax > 0:
            ok &= int(np.abs(codes[r]).max()) == 127
    # ties at exact midpoints (scale 2^-3: amax 127 / 8)
    row = np.zeros(192, np.float32)
    row[0] = 127 / 8
    row[1:7] = np.array([2.5, 3.5, -2.5, -3.5, 0.5, -0.5], np.float32) / 8
    c, sc = prefill_ref.quantize_rows_int8(_bf16_bits(row[None]))
    ok &= sc[0] == np.float32(1 / 8)
    ok &= list(c[0, :7]) == [127, 2, 4, -2, -4, 0, 0]
    return bool(ok)


def check_k_codes_are_nearest_per_block():
    case = make_prefill_case(seqlens=[200, 3], num_heads=2, seed=9)
    case.k[5, 1] = 0x4700                           # one large key in block 0, head 1
    case.k[128:200, 0] = 0                          # an all-zero block of head 0
    codes, scales = prefill_ref.quantize_k_blocks(case.k, case.cu_seqlens)
    x = oracle.decode_bf16(case.k).astype(np.float32)
    ok = scales.shape == (3, 2)
    cand = np.arange(-127, 128)
    for bi, (t0, t1) in enumerate([(0, 128), (128, 200), (200, 203)]):
        for h in range(2):
            amax = np.float32(np.abs(x[t0:t1, h]).max())
            want = np.float32(amax / np.float32(127)) if amax > 0 else np.float32(1)
            ok &= scales[bi, h] == want
            y = (x[t0:t1, h] / want).astype(np.float32).astype(np.float64).ravel()
            sub = np.linspace(0, y.size - 1, 300).astype(int)       # a sample, plus the max
            sub = np.append(sub, np.argmax(np.abs(y)))
            d = np.abs(y[sub][:, None] - cand[None, :])
            for row, j in enumerate(sub):
                ties = cand[d[row] == d[row].min()]
                want_c = ties[0] if len(ties) == 1 else ties[ties % 2 == 0][0]
                ok &= int(codes[t0:t1, h].ravel()[j]) == int(want_c)
            if amax > 0:
                ok &= int(np.abs(codes[t0:t1, h]).max()) == 127
            else:
                ok &= not codes[t0:t1, h].any()
    return bool(ok)


def check_v_codes_are_nearest_per_block_and_channel():
    case = make_prefill_case(seqlens=[300, 2], num_heads=2, seed=6)
    case.v[:, 1, 5] = 0                                  # an all-zero channel
    codes, scales = prefill_ref.quantize_v_blocks(case.v, case.cu_seqlens)
    x = oracle.decode_bf16(case.v).astype(np.float32)
    fin = E4M3_VALUES[FINITE].astype(np.float64)
    fcodes = np.arange(256)[FINITE]
    ok = scales.shape == (3 + 1, 2, 128)
    blocks = [(0, 128), (128, 256), (256, 300), (300, 302)]
    for bi, (t0, t1) in enumerate(blocks):
        for h in range(2):
            amax = np.abs(x[t0:t1, h]).max(0).astype(np.float64)
            # the smallest power of two that brings the channel within 448, by search
            want = np.ones(128)
            for c in range(128):
                if amax[c] > 0:
                    e = -127
                    while amax[c] / 2.0 ** e > 448:
                        e += 1
                    want[c] = 2.0 ** e
            ok &= np.array_equal(scales[bi, h].astype(np.float64), want)
            for c in (0, 5, 77):
                y = np.clip(x[t0:t1, h, c].astype(np.float64) / want[c], -448, 448)
                for j, yy in enumerate(y.astype(np.float64)):
                    d = np.abs(fin - yy)
                    ties = fcodes[d == d.min()]
                    if len(ties) > 1:
                        ties = ties[ties % 2 == 0]
                        if yy == 0:
                            ties = ties[(ties & 0x80) == (0x80 if np.signbit(yy) else 0)]
                    ok &= int(codes[t0 + j, h, c]) == int(ties[0])
            m = np.abs(oracle.decode_e4m3(codes[t0:t1, h])).max(0)
            ok &= bool(np.all(((m >= 224) & (m <= 448)) | (amax == 0)))
    return bool(ok)


def check_p_quantizer():
    p = np.array([1.0, 0.5, 1 / 448, 2.0 ** -12, 0.0, 0.3, 0.999])
    got = prefill_ref.quantize_p(p)
    fin = np.sort(np.abs(E4M3_VALUES[FINITE]))
    ok = got[0] == 1.0 and got[1] == 0.5 and got[4] == 0.0
    for i, pp in enumerate(p):
        y = pp * 448
        near = fin[np.argmin(np.abs(fin - y))]
        ok &= abs(got[i] * 448 - y) <= abs(near - y) + 1e-15
    return bool(ok)


CHECKS = [check_exact_inputs_quantize_exactly, check_blocked_softmax_is_plain_softmax,
          check_pipeline_is_causal_attention_up_to_p_rounding,
          check_first_token_and_zero_query_closed_forms, check_int8_codes_are_nearest_brute_force,
          check_k_codes_are_nearest_per_block, check_v_codes_are_nearest_per_block_and_channel,
          check_p_quantizer]


@pytest.mark.parametrize("check", CHECKS, ids=[c.__name__ for c in CHECKS])
def test_prefill_pin(check):
    assert check()


def _pins_pass():
    for c in CHECKS:
        try:
            if not c():
                return False
        except Exception:
            return False
    return True


ORIG_INT8 = prefill_ref.quantize_rows_int8
ORIG_K = prefill_ref.quantize_k_blocks
ORIG_V = prefill_ref.quantize_v_blocks
ORIG_P = prefill_ref.quantize_p
ORIG_ROW = prefill_ref.blocked_attend_row


def _mut_int8_over_128(x):
    c, s = ORIG_INT8(x)
    return c, (s * np.float32(127 / 128)).astype(np.float32)


def _mut_int8_truncate(x):
    xf = prefill_ref._f32(x)
    _, s = ORIG_INT8(x)
    return np.clip(np.trunc(xf / s[..., None]), -127, 127).astype(np.int8), s


def _mut_v_per_token(v, cu):
    codes, scales = ORIG_V(v, cu)
    return codes, np.full_like(scales, scales.mean())


def _mut_v_scale_not_pow2(v, cu):
    # the plain max / 448 scale in place of the power of two
    x = prefill_ref._f32(v)
    codes, scales = ORIG_V(v, cu)
    blocks = prefill_ref._blocks(cu)
    for bi, (t0, t1) in enumerate(blocks):
        amax = np.abs(x[t0:t1]).max(0)
        sc = np.where(amax > 0, (amax / np.float32(448)).astype(np.float32), np.float32(1))
        scales[bi] = sc
        codes[t0:t1] = prefill_ref.encode_e4m3(np.clip((x[t0:t1] / sc).astype(np.float32), -448, 448))
    return codes, scales


def _mut_k_first_token_scale(k, cu):
    # the block's scale taken from its first token only
    x = prefill_ref._f32(k)
    codes, scales = ORIG_K(k, cu)
    for bi, (t0, t1) in enumerate(prefill_ref._blocks(cu)):
        sc = (np.abs(x[t0]).max(-1) / np.float32(127)).astype(np.float32)
        sc = np.where(sc > 0, sc, np.float32(1))
        scales[bi] = sc
        codes[t0:t1] = np.clip(np.rint(x[t0:t1] / sc[None, :, None]), -127, 127).astype(np.int8)
    return codes, scales


def _mut_p_not_divided(p):
    return ORIG_P(p) * 448.0


def _mut_no_acc_rescale(s, values, quant_p=True, block=prefill_ref.KEY_BLOCK):
    n = s.shape[0]
    m, l, acc = -np.inf, 0.0, np.zeros(values.shape[1])
    for b0 in range(0, n, block):
        sb = s[b0:b0 + block]
        m_new = max(m, float(sb.max()))
        alpha = np.exp(m - m_new)
        p = np.exp(sb - m_new)
        l = l * alpha + float(p.sum())
        pu = prefill_ref.quantize_p(p) if quant_p else p
        acc = acc + pu @ values[b0:b0 + block]
        m = m_new
    return acc / l, m + np.log(l)


def _mut_lse_log2(s, values, quant_p=True, block=prefill_ref.KEY_BLOCK):
    o, lse = ORIG_ROW(s, values, quant_p, block)
    m = float(s.max())
    return o, m + math.log2(math.exp(lse - m))


def _mut_first_block_only(s, values, quant_p=True, block=prefill_ref.KEY_BLOCK):
    return ORIG_ROW(s[:block], values[:block], quant_p, block)


@pytest.mark.parametrize("name,mutant", [
    ("quantize_rows_int8", _mut_int8_over_128), ("quantize_rows_int8", _mut_int8_truncate),
    ("quantize_v_blocks", _mut_v_per_token), ("quantize_v_blocks", _mut_v_scale_not_pow2),
    ("quantize_k_blocks", _mut_k_first_token_scale), ("quantize_p", _mut_p_not_divided),
    ("blocked_attend_row", _mut_no_acc_rescale), ("blocked_attend_row", _mut_lse_log2),
    ("blocked_attend_row", _mut_first_block_only)])
def test_planted_prefill_mistakes_are_caught(monkeypatch, name, mutant):
    assert _pins_pass()
    monkeypatch.setattr(prefill_ref, name, mutant)
    assert not _pins_pass()

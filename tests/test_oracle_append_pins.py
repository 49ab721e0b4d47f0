"""Pins of the cache-append oracle (``oracle/append_ref.py``) against things
other than itself (CPU only): the format's own values and midpoints, the
library cast ``torch.float8_e4m3fn``, the round-trip error bound of a 3-bit
mantissa, and the decode oracle's gather reading the appended rows back.
``test_planted_append_mistakes_are_caught`` plants plausible mistakes in the
oracle and checks that some pin fails.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import append_ref
from workloads import make_case

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

FINITE = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)


def _bf16(x):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _f32(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ------------------------------------------------------------------ encoder

def check_encoder_inverts_every_finite_code():
    vals = oracle.decode_e4m3(FINITE)
    return np.array_equal(append_ref.encode_e4m3(vals), FINITE)


def check_midpoints_go_to_the_even_code():
    codes = np.arange(0x00, 0x7E, dtype=np.uint8)            # pairs (c, c + 1), c + 1 <= 0x7E
    lo, hi = oracle.decode_e4m3(codes), oracle.decode_e4m3(codes + 1)
    mid = (lo + hi) / 2                                         # exact in float64
    even = np.where(codes % 2 == 0, codes, codes + 1).astype(np.uint8)
    ok = np.array_equal(append_ref.encode_e4m3(mid), even)
    ok &= np.array_equal(append_ref.encode_e4m3(-mid), even | 0x80)
    # just off the midpoint the nearer code wins
    step = hi - lo
    ok &= np.array_equal(append_ref.encode_e4m3(mid - step / 64), codes)
    ok &= np.array_equal(append_ref.encode_e4m3(mid + step / 64), codes + 1)
    return bool(ok)


def check_encoder_matches_torch_cast():
    rng = np.random.default_rng(11)
    mag = np.exp2(rng.uniform(-14.0, np.log2(448.0), 200_000)).astype(np.float32)
    y = np.where(rng.random(mag.size) < 0.5, -mag, mag).astype(np.float32)
    y = np.concatenate([y, np.float32([0.0, -0.0, 448.0, -448.0, 2.0 ** -9, 2.0 ** -10,
                                       1.5 * 2.0 ** -9, 2.0 ** -6])])
    lib = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return np.array_equal(append_ref.encode_e4m3(y.astype(np.float64)), lib)


def test_encoder_inverts_every_finite_code():
    assert check_encoder_inverts_every_finite_code()


def test_midpoints_go_to_the_even_code():
    assert check_midpoints_go_to_the_even_code()


def test_encoder_matches_torch_cast():
    assert check_encoder_matches_torch_cast()


def test_encoder_rejects_out_of_range():
    with pytest.raises(ValueError):
        append_ref.encode_e4m3(np.array([449.0]))
    with pytest.raises(ValueError):
        append_ref.encode_e4m3(np.array([np.nan]))


# ------------------------------------------------------------------ per-token quantization

def _rows():
    rng = np.random.default_rng(5)
    rows = [rng.normal(0, s, 576) for s in (0.5, 1e-3, 40.0)]
    rows.append(np.zeros(576))
    one = np.zeros(576)
    one[17] = -3.25
    rows.append(one)
    rows.append(rng.normal(0, 1, 576) * np.exp2(rng.integers(-20, 8, 576)))   # wide spread
    return _bf16(np.stack(rows))


def check_row_quantization():
    bits = _rows()
    x = _f32(bits)
    codes, scale = append_ref.quantize_rows_e4m3(x)
    ok = True
    amax = np.abs(x).max(axis=-1)
    want = np.where(amax > 0, (amax / np.float32(448)).astype(np.float32), np.float32(1.0))
    ok &= np.array_equal(scale, want.astype(np.float32))
    for r in range(x.shape[0]):
        if amax[r] == 0:
            ok &= bool(np.all(codes[r] == 0))
            continue
        # the largest element takes the largest code magnitude
        ok &= int(codes[r, np.argmax(np.abs(x[r]))]) & 0x7F == 0x7E
        # within half a code step of x / s, for the value the code decodes to
        y = x[r].astype(np.float64) / float(scale[r])
        dec = oracle.decode_e4m3(codes[r])
        a = np.abs(y)
        e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
        half_step = np.exp2(e - 4)
        ok &= bool(np.all(np.abs(dec - y) <= half_step * (1 + 1e-6)))
        ok &= bool(np.all((np.signbit(dec) == np.signbit(y)) | (dec == 0)))
    return bool(ok)


def test_row_quantization():
    assert check_row_quantization()


# ------------------------------------------------------------------ placement

def _append_case(kv_dtype):
    # a cache holding every sequence's tokens; the last n_b rows of each are
    # wiped (NaN) and then appended back
    kv_lens, new = [70, 5, 129, 64, 3], [2, 5, 1, 0, 3]
    case = make_case(kv_lens=kv_lens, q_lens=[1] * 5, seed=41, kv_dtype="bf16",
                     page_size=16 if kv_dtype == "bf16" else 64, num_heads=8)
    P = case.page_size
    max_new = max(new)
    rows = np.zeros((5, max_new, 576), np.uint16)
    wiped = case.kv.copy()
    for b, n in enumerate(new):
        for t in range(n):
            p = kv_lens[b] - n + t
            page, slot = case.block_table[b, p // P], p % P
            rows[b, t] = case.kv[page, slot]
            wiped[page, slot] = 0x7FC0
    return case, np.array(new, np.int32), rows, wiped


def check_bf16_append_reads_back():
    case, new, rows, wiped = _append_case("bf16")
    kv, _, skipped = append_ref.kv_append_ref(wiped, None, case.block_table, case.kv_lens, new,
                                              rows, case.page_size, "bf16")
    ok = skipped == 0 and np.array_equal(kv, case.kv)
    for b in range(case.batch):
        L = int(case.kv_lens[b])
        got = oracle.gather_latent(kv, case.block_table[b], L, case.page_size, "bf16")
        ok &= np.array_equal(got[L - new[b]:], oracle.decode_bf16(rows[b, :new[b]]))
    return bool(ok)


def check_e4m3_append_reads_back():
    case, new, rows, _ = _append_case("fp8_e4m3")
    pages = case.kv.shape[0]
    kv0 = np.full((pages, case.page_size, 576), 0x7F, np.uint8)    # NaN codes
    sc0 = np.full((pages, case.page_size), np.nan, np.float32)
    kv, sc, skipped = append_ref.kv_append_ref(kv0, sc0, case.block_table, case.kv_lens, new,
                                               rows, case.page_size, "fp8_e4m3")
    ok = skipped == 0
    n_written = 0
    for b in range(case.batch):
        L, n = int(case.kv_lens[b]), int(new[b])
        n_pages = (L + case.page_size - 1) // case.page_size
        flat = kv[case.block_table[b, :n_pages]].reshape(-1, 576)[:L]
        fsc = sc[case.block_table[b, :n_pages]].reshape(-1)[:L]
        x = _f32(rows[b, :n]).astype(np.float64)
        dec = oracle.decode_e4m3(flat[L - n:]) * fsc[L - n:, None].astype(np.float64)
        # within half a code step (relative 2^-4) of normal values, 2^-10 s below
        tol = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * fsc[L - n:, None]) * (1 + 1e-6)
        ok &= bool(np.all(np.abs(dec - x) <= tol))
        ok &= bool(np.all(flat[: L - n] == 0x7F))                   # older rows untouched
        n_written += n
    ok &= int(np.sum(kv != 0x7F)) <= n_written * 576
    ok &= int(np.sum(~np.isnan(sc))) == n_written
    return bool(ok)


def check_out_of_pool_rows_are_skipped():
    case, new, rows, wiped = _append_case("bf16")
    bt = case.block_table.copy()
    P = case.page_size
    bt[0, (int(case.kv_lens[0]) - 1) // P] = -1                   # page of seq 0's new tokens
    bt[2, (int(case.kv_lens[2]) - 1) // P] = case.kv.shape[0]     # past the pool
    kv_lens = case.kv_lens.copy()
    kv_lens[4] = 1                                                 # 3 new tokens, position -2, -1, 0
    kv, _, skipped = append_ref.kv_append_ref(wiped, None, bt, kv_lens, new, rows, P, "bf16")
    ok = skipped == 2 + 1 + 2          # both tokens of seq 0 sit on the removed page
    ok &= np.array_equal(kv[bt[4, 0], 0], rows[4, 2])
    for b, p in ((0, 68), (0, 69), (2, 128)):                       # not written
        page = case.block_table[b, p // P]
        ok &= np.array_equal(kv[page, p % P], wiped[page, p % P])
    # a sequence that claims more new tokens than max_new: every row skipped
    too_many = new.copy()
    too_many[1] = rows.shape[1] + 1
    _, _, sk2 = append_ref.kv_append_ref(wiped, None, case.block_table, case.kv_lens, too_many,
                                         rows, P, "bf16")
    ok &= sk2 == rows.shape[1]
    return bool(ok)


def test_bf16_append_reads_back():
    assert check_bf16_append_reads_back()


def test_e4m3_append_reads_back():
    assert check_e4m3_append_reads_back()


def test_out_of_pool_rows_are_skipped():
    assert check_out_of_pool_rows_are_skipped()


# ------------------------------------------------------------------ planted mistakes

CHECKS = [check_encoder_inverts_every_finite_code, check_midpoints_go_to_the_even_code,
          check_encoder_matches_torch_cast, check_row_quantization, check_bf16_append_reads_back,
          check_e4m3_append_reads_back, check_out_of_pool_rows_are_skipped]


def _pins_pass():
    for c in CHECKS:
        try:
            if not c():
                return False
        except Exception:
            return False
    return True


ORIG_ENCODE = append_ref.encode_e4m3
ORIG_QUANT = append_ref.quantize_rows_e4m3
ORIG_POS = append_ref.append_positions


def _mut_ties_to_odd(y):
    y = np.asarray(y, np.float64)
    vals, codes = append_ref._TABLE
    a = np.abs(y)
    hi = np.clip(np.searchsorted(vals, a, side="left"), 0, len(vals) - 1)
    lo = np.clip(hi - 1, 0, len(vals) - 1)
    d_lo, d_hi = a - vals[lo], vals[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((codes[hi] & 1) == 1))
    mag = np.where(pick_hi, codes[hi], codes[lo]).astype(np.uint8)
    return np.where(np.signbit(y), mag | 0x80, mag).astype(np.uint8)


def _mut_truncate(y):
    y = np.asarray(y, np.float64)
    vals, codes = append_ref._TABLE
    idx = np.clip(np.searchsorted(vals, np.abs(y), side="right") - 1, 0, len(vals) - 1)
    return np.where(np.signbit(y), codes[idx] | 0x80, codes[idx]).astype(np.uint8)


def _mut_drop_sign(y):
    return ORIG_ENCODE(np.abs(np.asarray(y, np.float64)))


def _mut_scale_127(x):
    x = np.asarray(x, np.float32)
    amax = np.max(np.abs(x), axis=-1)
    s = np.where(amax > 0, amax / np.float32(127), 1).astype(np.float32)
    y = np.clip(x / s[..., None], -448, 448)
    return ORIG_ENCODE(y), s


def _mut_scale_mean(x):
    x = np.asarray(x, np.float32)
    amax = np.mean(np.abs(x), axis=-1) * 3
    s = np.where(amax > 0, amax / np.float32(448), 1).astype(np.float32)
    y = np.clip(x / s[..., None], -448, 448)
    return ORIG_ENCODE(y), s


def _mut_pos_off_by_one(kv_lens, new_lens, max_new, block_table, page_size, num_pages):
    out, sk = ORIG_POS(kv_lens, new_lens, max_new, block_table, page_size, num_pages)
    return [(b, t, page, (slot + 1) % page_size) for b, t, page, slot in out], sk


def _mut_pos_from_start(kv_lens, new_lens, max_new, block_table, page_size, num_pages):
    zero = np.array([int(new_lens[b]) if new_lens is not None else max_new
                     for b in range(len(kv_lens))])
    return ORIG_POS(zero, new_lens, max_new, block_table, page_size, num_pages)


def _mut_no_skip(kv_lens, new_lens, max_new, block_table, page_size, num_pages):
    out, _ = ORIG_POS(kv_lens, new_lens, max_new, block_table, page_size, num_pages)
    return out, 0


@pytest.mark.parametrize("target,mutant", [
    ("encode_e4m3", _mut_ties_to_odd),
    ("encode_e4m3", _mut_truncate),
    ("encode_e4m3", _mut_drop_sign),
    ("quantize_rows_e4m3", _mut_scale_127),
    ("quantize_rows_e4m3", _mut_scale_mean),
    ("append_positions", _mut_pos_off_by_one),
    ("append_positions", _mut_pos_from_start),
    ("append_positions", _mut_no_skip),
])
def test_planted_append_mistakes_are_caught(monkeypatch, target, mutant):
    assert _pins_pass()
    monkeypatch.setattr(append_ref, target, mutant)
    assert not _pins_pass()

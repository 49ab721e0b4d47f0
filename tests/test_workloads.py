"""Checks of the seeded input recipe (CPU only)."""
import math

import numpy as np
import pytest

from workloads import make_case, workload


def test_tiny_fp32_recipe():
    c = workload("tiny_fp32")
    assert c.batch == 2 and c.num_heads == 8 and c.d_qk == 80 and c.d_latent == 64
    assert list(c.kv_lens) == [37, 128] and c.page_size == 16
    assert abs(c.sm_scale - 1 / math.sqrt(80)) < 1e-15
    assert c.kv.dtype == np.float32


def test_same_seed_same_bits():
    a = workload("v3_decode_bf16", batch_override=4)
    b = workload("v3_decode_bf16", batch_override=4)
    assert np.array_equal(a.kv, b.kv) and np.array_equal(a.q, b.q)
    assert np.array_equal(a.block_table, b.block_table)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8_e4m3"])
def test_poison_layout(kv_dtype):
    c = make_case(kv_lens=[70, 64, 1], q_lens=[1, 2, 1], max_q_len=2, num_heads=4,
                  d_latent=32, d_rope=8, page_size=64, kv_dtype=kv_dtype, seed=3)
    nan_code = 0x7FC0 if kv_dtype == "bf16" else 0x7F
    used = set()
    for b, L in enumerate(c.kv_lens):
        n = (int(L) + 63) // 64
        pages = c.block_table[b, :n]
        used.update(pages.tolist())
        assert np.all(c.block_table[b, n:] == -1)
        rows = c.kv[pages].reshape(-1, c.d_qk)
        assert not np.any(rows[:L] == nan_code) or kv_dtype == "fp8_e4m3"
        assert np.all(rows[L:] == nan_code)
    spare = sorted(set(range(c.num_pages)) - used)
    assert len(spare) >= 8
    assert np.all(c.kv[spare] == nan_code)
    # padded query rows are NaN bf16
    assert np.all(c.q[0, 1] == 0x7FC0) and np.all(c.q[2, 1] == 0x7FC0)
    if kv_dtype == "fp8_e4m3":
        assert np.all(np.isnan(c.kv_scale[spare]))
        s = c.kv_scale[c.block_table[0, 0]]
        assert np.all(s > 0)


def test_named_length_ranges():
    c = workload("mtp_verify_bf16", batch_override=16)
    assert np.all((c.kv_lens >= 512) & (c.kv_lens <= 8192)) and np.all(c.q_lens == 2)
    r = workload("ragged_serving_bf16", batch_override=32)
    assert np.all((r.kv_lens >= 64) & (r.kv_lens <= 32768))
    assert (r.q_lens == 2).sum() == 16 and (r.q_lens == 1).sum() == 16

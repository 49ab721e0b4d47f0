"""Seeded synthetic inputs for the cache-append tests (CPU emulator and GPU):
a paged pool filled with random bytes, a permuted block table and the new
tokens' bf16 rows.  Input generation only: no append arithmetic lives here.
"""
import numpy as np
import torch


def _bf16_bits(x):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


N_SPECIAL = 7


def special_rows(n_rows, rng):
    """Rows that reach every path of the quantizer: all zero, one spike, x/s on
    exact midpoints between codes (s = 1), the subnormal range, wide spreads,
    scales on both sides of 2^-64, bf16 subnormal inputs; then random rows."""
    rows = []
    z = np.zeros(576, np.float32)
    rows.append(z)
    one = z.copy()
    one[300] = -7.0
    rows.append(one)
    ties = z.copy()
    ties[0] = 448.0                                   # scale exactly 1
    mids = [1.0625, 1.1875, 2.125, 0.0087890625, 0.001953125 * 1.5, 0.001953125 * 0.5,
            0.015625 * 0.9375, 240.0, 416.0, 1.0 / 1024]
    for i, m in enumerate(mids):
        ties[1 + 2 * i] = m
        ties[2 + 2 * i] = -m
    rows.append(ties)
    rows.append((rng.standard_normal(576) * np.exp2(rng.integers(-24, 10, 576))).astype(np.float32))
    # scales below 2^-64 (a true division in the kernel), and just above it
    rows.append((rng.standard_normal(576) * 1e-19).astype(np.float32))
    rows.append((rng.standard_normal(576) * 2e-17).astype(np.float32))
    # bf16 subnormals next to a normal maximum
    sub = (rng.standard_normal(576) * 1e-39).astype(np.float32)
    sub[5] = 3.0
    rows.append(sub)
    while len(rows) < n_rows:
        rows.append((rng.standard_normal(576) * rng.choice([0.5, 1e-3, 30.0])).astype(np.float32))
    return _bf16_bits(np.stack(rows[:n_rows]))


def make_append_case(kv_lens, new_lens, page_size, kv_dtype, seed, max_new=None, spare=3):
    rng = np.random.default_rng(seed)
    kv_lens = np.asarray(kv_lens, np.int32)
    new_lens = np.asarray(new_lens, np.int32)
    B = len(kv_lens)
    max_new = int(max_new if max_new is not None else max(1, new_lens.max()))
    n_pages = [(int(L) + page_size - 1) // page_size for L in kv_lens]
    max_pages = max(1, max(n_pages))
    pool = sum(n_pages) + spare
    perm = rng.permutation(pool).astype(np.int32)
    bt = np.full((B, max_pages), -1, np.int32)
    k = 0
    for b, n in enumerate(n_pages):
        bt[b, :n] = perm[k:k + n]
        k += n
    if kv_dtype == "bf16":
        kv = rng.integers(0, 1 << 16, (pool, page_size, 576), dtype=np.uint16)
        sc = None
    else:
        kv = rng.integers(0, 256, (pool, page_size, 576), dtype=np.uint8)
        sc = rng.standard_normal((pool, page_size)).astype(np.float32)
    rows = special_rows(B * max_new, rng).reshape(B, max_new, 576)
    # the special rows go to the first new tokens that are written
    specials = special_rows(N_SPECIAL, rng)
    k = 0
    for b in range(B):
        for t in range(min(int(new_lens[b]), max_new)):
            if k < N_SPECIAL:
                rows[b, t] = specials[k]
                k += 1
    return dict(kv=kv, kv_scale=sc, block_table=bt, kv_lens=kv_lens, new_lens=new_lens,
                new_rows_bits=rows, page_size=page_size, kv_dtype=kv_dtype)

"""Seeded synthetic inputs for absorbed-MLA paged decode.

This module only draws random numbers and lays them out in the paged format.
It holds none of the attention arithmetic: the float64 oracle (``oracle/``) and
the HIP path both consume what it produces, and neither imports the other.

Rounding to storage formats uses library casts only (``torch.bfloat16`` for
round-to-nearest-even bf16, ``torch.float8_e4m3fn`` for OCP E4M3), so no codec
logic is shared with the oracle, which decodes the stored bits itself.

Recipe (one ``numpy.random.default_rng(seed)`` stream, drawn in this order):
kv_lens -> q_lens -> page permutation -> Q -> KV -> (fp8 per-token quantisation).

* Q  ~ N(0, 1) rounded to bf16 (fp32 for the tiny fp32 case).
* KV ~ kv_std * N(0, 1) rounded to bf16, or quantised to e4m3 with one fp32
  scale per cached token: scale = amax(|row|) / 448, code = RNE(row / scale),
  saturated to +-448 (the per-token symmetric convention, zero-point 0).
* The page pool holds sum_b ceil(L_b / P) used pages plus max(8, 2 %) spare
  pages; pages are placed by a random permutation of the pool.
* Spare pages, page tails past kv_len and padded query rows (t >= q_len[b])
  are NaN, so any read of them poisons the result.
* Unused block-table entries are -1 (callers may re-poison them).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

BF16_NAN = np.uint16(0x7FC0)
E4M3_NAN = np.uint8(0x7F)


@dataclass
class MLACase:
    """One decode call's inputs, as raw storage bits plus metadata."""

    name: str
    batch: int
    num_heads: int
    d_latent: int
    d_rope: int
    page_size: int
    kv_dtype: str                 # "bf16" | "fp8_e4m3" | "fp32"
    causal: bool
    sm_scale: float
    kv_lens: np.ndarray           # [B] int32
    q_lens: np.ndarray            # [B] int32
    block_table: np.ndarray       # [B, max_pages] int32
    q: np.ndarray                 # [B, q_max, H, D] uint16 bf16 bits (float32 for fp32)
    kv: np.ndarray                # [num_pages, P, D] uint16 / uint8 / float32
    kv_scale: Optional[np.ndarray] = None   # [num_pages, P] float32 (fp8 only)
    meta: dict = field(default_factory=dict)

    @property
    def d_qk(self) -> int:
        return self.d_latent + self.d_rope

    @property
    def max_q_len(self) -> int:
        return int(self.q.shape[1])

    @property
    def num_pages(self) -> int:
        return int(self.kv.shape[0])

    @property
    def max_pages(self) -> int:
        return int(self.block_table.shape[1])


def _to_bf16_bits(x: np.ndarray) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _to_e4m3_per_token(x: np.ndarray):
    """Per-token symmetric e4m3 quantisation of rows of ``x`` (float32)."""
    import torch
    x = np.ascontiguousarray(x, dtype=np.float32)
    amax = np.abs(x).max(axis=-1).astype(np.float32)
    scale = (amax / np.float32(448.0)).astype(np.float32)
    scale = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    y = np.clip(x / scale[..., None], -448.0, 448.0).astype(np.float32)
    codes = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, scale


def make_case(*, name: str = "custom", kv_lens, q_lens=None, num_heads: int = 128,
              d_latent: int = 512, d_rope: int = 64, page_size: int = 64,
              kv_dtype: str = "bf16", causal: bool = True, sm_scale: Optional[float] = None,
              seed: int = 0, kv_std: float = 0.5, q_std: float = 1.0,
              max_q_len: Optional[int] = None, extra_pages_per_seq: int = 0,
              rng: Optional[np.random.Generator] = None) -> MLACase:
    """Lay out a paged-cache decode call for explicit per-sequence lengths."""
    rng = rng if rng is not None else np.random.default_rng(seed)
    kv_lens = np.asarray(kv_lens, dtype=np.int32)
    B = int(kv_lens.shape[0])
    q_lens = np.ones(B, np.int32) if q_lens is None else np.asarray(q_lens, dtype=np.int32)
    q_max = int(max_q_len if max_q_len is not None else max(1, int(q_lens.max(initial=1))))
    D = d_latent + d_rope
    P = int(page_size)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)

    n_pages = [(int(L) + P - 1) // P for L in kv_lens]
    used = int(sum(n_pages))
    spare = max(8, int(math.ceil(0.02 * used)))
    num_pages = used + spare
    perm = rng.permutation(num_pages).astype(np.int32)
    max_pages = max(1, max(n_pages, default=1) + extra_pages_per_seq)
    block_table = np.full((B, max_pages), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(n_pages):
        block_table[b, :n] = perm[off:off + n]
        off += n

    qf = rng.standard_normal((B, q_max, num_heads, D), dtype=np.float32)
    if q_std != 1.0:
        qf *= np.float32(q_std)
    for b in range(B):
        qf[b, int(q_lens[b]):] = np.nan

    total = int(kv_lens.sum())
    kvf = rng.standard_normal((total, D), dtype=np.float32)
    if kv_std != 1.0:
        kvf *= np.float32(kv_std)

    # logical token index -> (physical page, slot)
    phys = np.empty(total, dtype=np.int64)
    off = 0
    for b in range(B):
        L = int(kv_lens[b])
        j = np.arange(L, dtype=np.int64)
        phys[off:off + L] = block_table[b, j // P].astype(np.int64) * P + (j % P)
        off += L

    kv_scale = None
    if kv_dtype in ("bf16", "fp8_e4m3"):
        q = _to_bf16_bits(qf)
        for b in range(B):
            q[b, int(q_lens[b]):] = BF16_NAN
    if kv_dtype == "bf16":
        kv = np.full((num_pages * P, D), BF16_NAN, dtype=np.uint16)
        kv[phys] = _to_bf16_bits(kvf)
    elif kv_dtype == "fp8_e4m3":
        codes, scale = _to_e4m3_per_token(kvf)
        kv = np.full((num_pages * P, D), E4M3_NAN, dtype=np.uint8)
        kv[phys] = codes
        kv_scale = np.full(num_pages * P, np.nan, dtype=np.float32)
        kv_scale[phys] = scale
        kv_scale = kv_scale.reshape(num_pages, P)
    elif kv_dtype == "fp32":
        q = qf
        kv = np.full((num_pages * P, D), np.nan, dtype=np.float32)
        kv[phys] = kvf
    else:
        raise ValueError(f"unknown kv_dtype {kv_dtype!r}")
    kv = kv.reshape(num_pages, P, D)

    return MLACase(name=name, batch=B, num_heads=num_heads, d_latent=d_latent,
                   d_rope=d_rope, page_size=P, kv_dtype=kv_dtype, causal=causal,
                   sm_scale=float(sm_scale), kv_lens=kv_lens, q_lens=q_lens,
                   block_table=block_table, q=q, kv=kv, kv_scale=kv_scale,
                   meta=dict(seed=seed, spare_pages=spare, used_pages=used))


# --------------------------------------------------------------------------
# The five named workloads.  Lengths are drawn first from the same stream.
# --------------------------------------------------------------------------

def _lognormal_lengths(rng, n, mean, sigma, lo, hi):
    mu = math.log(mean) - sigma * sigma / 2.0
    x = rng.lognormal(mean=mu, sigma=sigma, size=n)
    return np.clip(np.rint(x), lo, hi).astype(np.int32)


WORKLOADS = {
    # name: (seed, description)
    "tiny_fp32": (1, "B 2, H 8, 64+16 / 64, kv_lens {37,128}, q 1, P 16, fp32, scale 1/sqrt(80)"),
    "v3_decode_bf16": (2, "B 64, H 128, 512+64, kv U[1024,4096], q 1, P 64, bf16, scale 1/sqrt(192)"),
    "mtp_verify_bf16": (3, "B 128, H 128, kv U[512,8192], q 2 causal, P 64, bf16"),
    "long_ctx_fp8": (4, "B 16, H 128, kv U[16384,32768], q 1, P 64, e4m3 KV + fp32 per-token scale"),
    "ragged_serving_bf16": (5, "256 seqs, log-normal kv (mean 2790, clip [64,32768]), half q 1 / half q 2, P 64, bf16"),
    "tree_verify_bf16": (6, "B 128, H 128, kv U[512,8192], 4 tree-shaped drafts (random branches), P 64, bf16"),
}


def workload(name: str, *, batch_override: Optional[int] = None) -> MLACase:
    """Build one named workload.  ``batch_override`` keeps the per-sequence
    length distribution but draws fewer sequences (for parity runs the oracle
    can finish quickly); ``None`` gives the full configuration."""
    seed, _ = WORKLOADS[name]
    rng = np.random.default_rng(seed)
    sm192 = 1.0 / math.sqrt(192.0)
    if name == "tiny_fp32":
        return make_case(name=name, kv_lens=[37, 128], q_lens=[1, 1], num_heads=8,
                         d_latent=64, d_rope=16, page_size=16, kv_dtype="fp32",
                         sm_scale=1.0 / math.sqrt(80.0), kv_std=1.0, rng=rng, seed=seed)
    if name == "v3_decode_bf16":
        B = batch_override or 64
        kv_lens = rng.integers(1024, 4096, size=B, endpoint=True).astype(np.int32)
        q_lens = np.ones(B, np.int32)
        return make_case(name=name, kv_lens=kv_lens, q_lens=q_lens, sm_scale=sm192,
                         rng=rng, seed=seed)
    if name == "mtp_verify_bf16":
        B = batch_override or 128
        kv_lens = rng.integers(512, 8192, size=B, endpoint=True).astype(np.int32)
        q_lens = np.full(B, 2, np.int32)
        return make_case(name=name, kv_lens=kv_lens, q_lens=q_lens, sm_scale=sm192,
                         rng=rng, seed=seed, causal=True)
    if name == "long_ctx_fp8":
        B = batch_override or 16
        kv_lens = rng.integers(16384, 32768, size=B, endpoint=True).astype(np.int32)
        q_lens = np.ones(B, np.int32)
        return make_case(name=name, kv_lens=kv_lens, q_lens=q_lens, sm_scale=sm192,
                         kv_dtype="fp8_e4m3", rng=rng, seed=seed)
    if name == "ragged_serving_bf16":
        B = batch_override or 256
        kv_lens = _lognormal_lengths(rng, B, 2790.0, 1.0, 64, 32768)
        q_lens = np.ones(B, np.int32)
        two = rng.choice(B, size=B // 2, replace=False)
        q_lens[two] = 2
        return make_case(name=name, kv_lens=kv_lens, q_lens=q_lens, sm_scale=sm192,
                         rng=rng, seed=seed, causal=True)
    if name == "tree_verify_bf16":
        # EAGLE-style drafts: 4 draft tokens per sequence on random branches
        B = batch_override or 128
        kv_lens = rng.integers(512, 8192, size=B, endpoint=True).astype(np.int32)
        q_lens = np.full(B, 4, np.int32)
        case = make_case(name=name, kv_lens=kv_lens, q_lens=q_lens, sm_scale=sm192,
                         rng=rng, seed=seed, causal=True)
        case.meta["tree_mask"] = tree_masks(q_lens, 4, "branch", seed=seed)
        return case
    raise KeyError(name)


def tree_masks(q_lens, max_q_len, kind, seed=0):
    """[B, max_q_len] uint32 mask words.  kind: causal (each token sees the
    drafts up to itself), diag (itself only), none (no draft), branch (token t
    sees itself and a random chain of earlier drafts: a random tree), random
    (any subset of the drafts, the token itself not always included)."""
    rng = np.random.default_rng(seed)
    B = len(q_lens)
    m = np.zeros((B, max_q_len), np.uint32)
    for b in range(B):
        q = int(q_lens[b])
        parent = [-1] * q
        for t in range(q):
            if kind == "causal":
                m[b, t] = (1 << (t + 1)) - 1
            elif kind == "diag":
                m[b, t] = 1 << t
            elif kind == "none":
                m[b, t] = 0
            elif kind == "branch":
                parent[t] = int(rng.integers(-1, t)) if t > 0 else -1
                word, p = 1 << t, parent[t]
                while p >= 0:
                    word |= 1 << p
                    p = parent[p]
                m[b, t] = word
            elif kind == "random":
                m[b, t] = int(rng.integers(0, 1 << q))
    return m

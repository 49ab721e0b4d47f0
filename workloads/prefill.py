"""Seeded synthetic inputs for the quantized causal prefill (random numbers
and layout only; none of the attention or quantization arithmetic).

Recipe (one ``numpy.random.default_rng(seed)`` stream, drawn in this order):
Q -> K -> V, each ``std * N(0, 1)`` in float32, then a per-channel offset
``k_bias * N(0, 1)`` added to every K row of a head (the shared channel
offset real keys carry; 0 by default), rounded to bf16 by ``torch.bfloat16``
(round to nearest even).  Sequences are packed along the token axis:
tokens cu_seqlens[s] .. cu_seqlens[s + 1] - 1 belong to sequence s.
Per head Q and K are 192 wide (128 + 64 rope) and V 128 wide (DeepSeek's
prefill head dims).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

D_QK = 192
D_V = 128


@dataclass
class PrefillCase:
    name: str
    seqlens: np.ndarray           # [S] int32
    cu_seqlens: np.ndarray        # [S + 1] int32
    num_heads: int
    sm_scale: float
    q: np.ndarray                 # [T, H, 192] uint16 bf16 bits
    k: np.ndarray                 # [T, H, 192] uint16
    v: np.ndarray                 # [T, H, 128] uint16
    meta: dict = field(default_factory=dict)
    d_qk: int = D_QK
    d_v: int = D_V

    @property
    def num_seqs(self) -> int:
        return int(len(self.seqlens))

    @property
    def num_tokens(self) -> int:
        return int(self.cu_seqlens[-1])


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def make_prefill_case(*, name: str = "custom", seqlens, num_heads: int = 16, seed: int = 0,
                      sm_scale: Optional[float] = None, q_std: float = 1.0, k_std: float = 1.0,
                      v_std: float = 1.0, k_bias: float = 0.0,
                      rng: Optional[np.random.Generator] = None) -> PrefillCase:
    rng = rng if rng is not None else np.random.default_rng(seed)
    seqlens = np.asarray(seqlens, dtype=np.int32)
    cu = np.concatenate([[0], np.cumsum(seqlens)]).astype(np.int32)
    T, H = int(cu[-1]), int(num_heads)

    def draw(shape, std):
        out = np.empty(shape, np.uint16)
        step = max(1, (1 << 24) // int(np.prod(shape[1:])))
        for t0 in range(0, shape[0], step):
            n = min(step, shape[0] - t0)
            x = rng.standard_normal((n,) + shape[1:], dtype=np.float32) * np.float32(std)
            out[t0:t0 + n] = _bf16_bits(x)
        return out

    q = draw((T, H, D_QK), q_std)
    if k_bias:
        kf = rng.standard_normal((T, H, D_QK), dtype=np.float32) * np.float32(k_std)
        bias = rng.standard_normal((1, H, D_QK), dtype=np.float32) * np.float32(k_bias)
        k = _bf16_bits(kf + bias)
    else:
        k = draw((T, H, D_QK), k_std)
    v = draw((T, H, D_V), v_std)
    scale = 1.0 / math.sqrt(D_QK) if sm_scale is None else float(sm_scale)
    return PrefillCase(name=name, seqlens=seqlens, cu_seqlens=cu, num_heads=H, sm_scale=scale,
                       q=q, k=k, v=v)


PREFILL_WORKLOADS = {
    # the page's long-input first-token case: one 64K-token prompt; 16 heads is
    # one GPU's share of DeepSeek's 128 under 8-way head parallelism
    "sage_prefill_64k": (7, "1 prompt x 65536 tokens, H 16, QK 192 / V 128, bf16 in, INT8 QK + FP8 PV"),
    # a mix of prompt lengths in one packed batch
    "sage_prefill_mix": (8, "8 prompts, lengths U[1024, 8192], H 16, QK 192 / V 128"),
}


def prefill_workload(name: str) -> PrefillCase:
    seed, _ = PREFILL_WORKLOADS[name]
    rng = np.random.default_rng(seed)
    if name == "sage_prefill_64k":
        return make_prefill_case(name=name, seqlens=[65536], num_heads=16, rng=rng)
    if name == "sage_prefill_mix":
        lens = rng.integers(1024, 8192, size=8, endpoint=True)
        return make_prefill_case(name=name, seqlens=lens, num_heads=16, rng=rng)
    raise KeyError(name)

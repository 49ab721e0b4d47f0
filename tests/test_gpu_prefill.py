"""Quantized prefill on the GPU (mla_prefill_quantize + mla_prefill_attn
through the C ABI): INT8 / e4m3 codes and scales bit-exact against the
oracle's quantizers; O and LSE against the oracle's blocked online softmax
at the e4m3 bar, on whole small cases and on sampled rows of a 64K-token
prompt."""

import numpy as np
import pytest

from tests.prefill_cases import check_attention, check_quantized
from workloads.prefill import PrefillCase, make_prefill_case, prefill_workload

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import mla_paged_decode_absorbed_amd as mla  # noqa: E402

DEV = "cuda"


def _bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(DEV)


def run_gpu(case):
    shape = mla.PrefillShape.make(case.seqlens, case.num_heads)
    cu = torch.from_numpy(case.cu_seqlens.astype(np.int32)).to(DEV)
    quant = mla.prefill_quantize(shape, cu, _bf16(case.q), _bf16(case.k), _bf16(case.v))
    out = torch.full((case.num_tokens, case.num_heads, 128), float("nan"), dtype=torch.bfloat16,
                     device=DEV)
    lse = torch.full((case.num_tokens, case.num_heads), 12345.0, dtype=torch.float32, device=DEV)
    mla.prefill_attn(shape, cu, quant, case.sm_scale, out=out, lse=lse)
    torch.cuda.synchronize()
    got = {"qc": quant.q_codes.cpu().numpy(), "qs": quant.q_scale.cpu().numpy(),
           "kc": quant.k_codes.cpu().numpy(), "ks": quant.k_scale.cpu().numpy(),
           "vc": quant.v_codes.cpu().numpy(), "vs": quant.v_scale.cpu().numpy(),
           "o": out.view(torch.int16).cpu().numpy().view(np.uint16), "lse": lse.cpu().numpy()}
    return got


@pytest.mark.parametrize("seqlens,H,seed", [
    ([300, 1, 5, 129], 2, 81),          # ragged tails, one-token sequence
    ([3, 0, 130], 1, 82),               # an empty sequence
    ([1000, 2048, 77], 16, 83),         # many key blocks, 16 heads (two per XCD)
    ([640], 8, 84),                     # exactly 5 blocks, no tail
])
def test_prefill_matches_oracle(seqlens, H, seed):
    case = make_prefill_case(seqlens=seqlens, num_heads=H, seed=seed)
    got = run_gpu(case)
    quant = check_quantized(case, got)
    T = case.num_tokens
    if T * H <= 4000:
        rows = None
    else:
        rng = np.random.default_rng(seed)
        rows = [(int(t), int(h)) for t, h in zip(rng.integers(0, T, 400), rng.integers(0, H, 400))]
        cu = case.cu_seqlens
        rows += [(int(cu[s]), 0) for s in range(case.num_seqs) if cu[s + 1] > cu[s]]
        rows += [(int(cu[s + 1]) - 1, H - 1) for s in range(case.num_seqs) if cu[s + 1] > cu[s]]
    check_attention(case, got["o"], got["lse"], rows=rows, quantized=quant)


def test_prefill_edge_values():
    case = make_prefill_case(seqlens=[140, 60], num_heads=3, seed=85, k_bias=2.0, v_std=0.01)
    case.q[7] = 0
    case.k[150, 1] = 0
    case.v[10:20, 2, 3] = 0
    case.q[20, 0, :] = 0x4480           # a peaky row: every element 1024
    case.q[21, 1, ::3] = 0xC480         # and -1024 in every third dim
    got = run_gpu(case)
    quant = check_quantized(case, got)
    check_attention(case, got["o"], got["lse"], quantized=quant)


def test_prefill_long_prompt_sampled():
    # the 64K-token prompt of the bench, 16 heads: every code of two heads
    # bit-exact, and sampled rows of those heads against the oracle
    case = prefill_workload("sage_prefill_64k")
    got = run_gpu(case)
    assert np.all(np.isfinite(got["lse"]))
    T = case.num_tokens
    rng = np.random.default_rng(86)
    for h in (0, 13):
        one = PrefillCase(name="one-head", seqlens=case.seqlens, cu_seqlens=case.cu_seqlens,
                          num_heads=1, sm_scale=case.sm_scale, q=case.q[:, h:h + 1],
                          k=case.k[:, h:h + 1], v=case.v[:, h:h + 1])
        sub = {"qc": got["qc"][:, h:h + 1], "qs": got["qs"][:, h:h + 1],
               "kc": got["kc"][:, h:h + 1], "ks": got["ks"][:, h:h + 1],
               "vc": got["vc"][:, h:h + 1], "vs": got["vs"][:, h:h + 1]}
        quant = check_quantized(one, sub)
        ts = [0, 127, 128, T - 1] + [int(t) for t in rng.integers(0, T, 6)]
        check_attention(one, got["o"][:, h:h + 1], got["lse"][:, h:h + 1],
                        rows=[(t, 0) for t in ts], quantized=quant)


def test_prefill_untouched_outside_rows():
    # sequences whose cu_seqlens entries run past T are not written
    case = make_prefill_case(seqlens=[130, 20], num_heads=2, seed=87)
    shape = mla.PrefillShape.make(case.seqlens, 2)
    bad_cu = torch.tensor([0, 130, 151], dtype=torch.int32, device=DEV)   # 151 > T = 150
    quant = mla.prefill_quantize(shape, bad_cu, _bf16(case.q), _bf16(case.k), _bf16(case.v))
    out = torch.full((150, 2, 128), 7.0, dtype=torch.bfloat16, device=DEV)
    lse = torch.full((150, 2), 12345.0, dtype=torch.float32, device=DEV)
    mla.prefill_attn(shape, bad_cu, quant, case.sm_scale, out=out, lse=lse)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy()
    assert np.all(o[130:] == 7.0) and np.all(lse[130:].cpu().numpy() == 12345.0)
    assert np.all(np.isfinite(lse[:130].cpu().numpy())) and not np.all(o[:130] == 7.0)

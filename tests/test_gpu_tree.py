"""Tree-shaped drafts on the GPU: a non-causal decode over the prefix merged
with the drafts by mla_tree_attend, against the tree oracle at the decode's
tolerances; a causal mask against the ordinary causal decode."""
import math

import numpy as np
import pytest

from oracle import tree_ref
from tests.tree_cases import tree_masks
from workloads import make_case

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import mla_paged_decode_absorbed_amd as mla  # noqa: E402
from tests.test_gpu_parity import LSE_TOL, TOL, run_gpu, shape_of, to_dev  # noqa: E402

DEV = "cuda"


def run_tree(case, mask, num_workgroups=None):
    q, kv, sc, bt, kvl, ql = to_dev(case)
    shape = shape_of(case)
    m = torch.from_numpy(mask.view(np.int32)).to(DEV)
    out, lse = mla.decode_tree(shape, q, kv, bt, case.kv_lens, case.q_lens, kvl, ql, m,
                               case.sm_scale, kv_scale=sc, num_workgroups=num_workgroups)
    torch.cuda.synchronize()
    return out, lse


def check_tree(case, mask, out, lse):
    O, L = tree_ref.mla_decode_tree_ref(case, mask)
    o = out.float().cpu().numpy().astype(np.float64)
    l = lse.cpu().numpy().astype(np.float64)
    mabs, mrel = TOL[case.kv_dtype]
    num = den = worst = 0.0
    for b in range(case.batch):
        q = int(case.q_lens[b])
        if q == 0:
            continue
        d = o[b, :q] - O[b, :q]
        assert np.all(np.isfinite(o[b, :q])), b
        worst = max(worst, float(np.abs(d).max()))
        num += float((d ** 2).sum())
        den += float((O[b, :q] ** 2).sum())
        same_inf = np.isinf(L[b, :q]) & (l[b, :q] == L[b, :q])
        dl = np.where(same_inf, 0.0, np.abs(l[b, :q] - L[b, :q]))
        assert float(dl.max()) <= LSE_TOL, (b, float(dl.max()))
    assert worst <= mabs, worst
    assert math.sqrt(num / max(den, 1e-300)) <= mrel


@pytest.mark.parametrize("kind", ["causal", "diag", "branch", "random", "none"])
def test_tree_masks(kind):
    case = make_case(kv_lens=[300, 8, 70, 4, 1000, 2500], q_lens=[4, 8, 3, 4, 0, 5], seed=61,
                     sm_scale=1 / math.sqrt(192), max_q_len=8)
    mask = tree_masks(case.q_lens, case.max_q_len, kind, seed=4)
    out, lse = run_tree(case, mask)
    check_tree(case, mask, out, lse)


@pytest.mark.parametrize("dtype,H", [("fp8_e4m3", 128), ("bf16", 16)])
def test_tree_dtypes_and_heads(dtype, H):
    case = make_case(kv_lens=[900, 4, 3000], q_lens=[4, 4, 2], seed=62, kv_dtype=dtype,
                     num_heads=H, sm_scale=1 / math.sqrt(192), max_q_len=4)
    mask = tree_masks(case.q_lens, case.max_q_len, "branch", seed=5)
    out, lse = run_tree(case, mask, num_workgroups=64)
    check_tree(case, mask, out, lse)


@pytest.mark.parametrize("H,qmax", [(20, 4), (8, 3), (128, 8)])
def test_tree_head_groups(H, qmax):
    case = make_case(kv_lens=[90, 3, 400, 5000], q_lens=[qmax, 3, 2, qmax], seed=64, num_heads=H,
                     sm_scale=1 / math.sqrt(192), max_q_len=qmax)
    mask = tree_masks(case.q_lens, case.max_q_len, "random", seed=7)
    out, lse = run_tree(case, mask)
    check_tree(case, mask, out, lse)


def test_causal_mask_matches_the_causal_decode():
    case = make_case(kv_lens=[700, 130, 2000], q_lens=[4, 2, 3], seed=63,
                     sm_scale=1 / math.sqrt(192), max_q_len=4)
    mask = tree_masks(case.q_lens, case.max_q_len, "causal")
    out_t, lse_t = run_tree(case, mask)
    (out_c, lse_c), _ = run_gpu(case)
    for b in range(case.batch):
        q = int(case.q_lens[b])
        d = (out_t[b, :q].float() - out_c[b, :q].float()).abs().max().item()
        assert d <= 2e-2
        assert (lse_t[b, :q] - lse_c[b, :q]).abs().max().item() <= 1e-3

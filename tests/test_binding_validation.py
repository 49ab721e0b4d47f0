"""The binding's size checks (no GPU): the C ABI takes bare device pointers,
so the Python layer rejects a tensor whose size or element type does not
match the shape struct before anything is launched.  Every case below fails
in the binding; none reaches the library."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import mla_paged_decode_absorbed_amd as mla  # noqa: E402

B, H, QMAX, P, NP, MAXP = 3, 16, 2, 64, 20, 5


def _shape(kvd=mla.KV_BF16):
    return mla.Shape.make(batch=B, num_heads=H, max_q_len=QMAX, page_size=P, num_pages=NP,
                          max_pages_per_seq=MAXP, kv_dtype=kvd)


def _tensors(kvd=mla.KV_BF16):
    fp8 = kvd == mla.KV_FP8_E4M3
    return dict(
        q=torch.zeros((B, QMAX, H, 576), dtype=torch.bfloat16),
        kv_cache=torch.zeros((NP, P, 576), dtype=torch.uint8 if fp8 else torch.bfloat16),
        block_table=torch.zeros((B, MAXP), dtype=torch.int32),
        kv_lens=torch.full((B,), 10, dtype=torch.int32),
        q_lens=torch.ones((B,), dtype=torch.int32),
        kv_scale=torch.ones((NP, P), dtype=torch.float32) if fp8 else None,
        out=torch.zeros((B, QMAX, H, 512), dtype=torch.bfloat16),
        lse=torch.zeros((B, QMAX, H), dtype=torch.float32))


class _NoLaunch(Exception):
    pass


@pytest.fixture
def no_launch(monkeypatch):
    """Any call past the binding's checks stops here instead of reaching the library."""
    def stop(*a, **k):
        raise _NoLaunch()
    for name in ("decode_fwd", "combine", "alloc_workspace", "load_library"):
        monkeypatch.setattr(mla, name, stop)


def _decode(kvd=mla.KV_BF16, **over):
    t = {**_tensors(kvd), **over}
    pl = mla.Plan(info=mla.PlanInfo(), host=None, device=None)
    return mla.decode(_shape(kvd), pl, t["q"], t["kv_cache"], t["block_table"], t["kv_lens"],
                      t["q_lens"], 0.07, kv_scale=t["kv_scale"], out=t["out"], lse=t["lse"])


def test_consistent_tensors_pass_the_checks(no_launch):
    with pytest.raises(_NoLaunch):
        _decode()
    with pytest.raises(_NoLaunch):
        _decode(mla.KV_FP8_E4M3)


@pytest.mark.parametrize("name,bad", [
    ("kv_cache", torch.zeros((NP - 1, P, 576), dtype=torch.bfloat16)),       # a page short
    ("kv_cache", torch.zeros((NP, P, 576), dtype=torch.float32)),            # wrong element
    ("block_table", torch.zeros((B, MAXP - 1), dtype=torch.int32)),
    ("block_table", torch.zeros((B, MAXP), dtype=torch.int64)),
    ("kv_lens", torch.zeros((B + 1,), dtype=torch.int32)),
    ("q_lens", torch.zeros((B - 1,), dtype=torch.int32)),
    ("out", torch.zeros((B, QMAX, H, 256), dtype=torch.bfloat16)),
    ("lse", torch.zeros((B, QMAX, H), dtype=torch.float16)),
    ("block_table", torch.zeros((MAXP, B), dtype=torch.int32).t()),           # not contiguous
])
def test_mismatched_tensor_is_rejected(no_launch, name, bad):
    with pytest.raises(ValueError, match=name):
        _decode(**{name: bad})


def test_e4m3_cache_needs_its_scales(no_launch):
    with pytest.raises(ValueError, match="kv_scale"):
        _decode(mla.KV_FP8_E4M3, kv_scale=None)
    with pytest.raises(ValueError, match="kv_scale"):
        _decode(mla.KV_FP8_E4M3, kv_scale=torch.ones((NP, P - 1), dtype=torch.float32))
    with pytest.raises(ValueError, match="kv_cache"):
        _decode(mla.KV_FP8_E4M3, kv_cache=torch.zeros((NP, P, 576), dtype=torch.bfloat16))


def test_check_and_tree_sizes(no_launch):
    t = _tensors()
    pl = mla.Plan(info=mla.PlanInfo(), host=None, device=None)
    with pytest.raises(ValueError, match="kv_lens"):
        mla.check(_shape(), pl, t["block_table"], torch.zeros(B + 2, dtype=torch.int32))
    with pytest.raises(ValueError, match="block_table"):
        mla.tree_attend(_shape(), t["q"], t["kv_cache"], t["block_table"][:, :2].contiguous(),
                        t["kv_lens"], t["q_lens"], torch.zeros((B, QMAX), dtype=torch.int32),
                        0.07, t["out"], t["lse"])


def test_prefill_sizes(monkeypatch):
    monkeypatch.setattr(mla, "load_library", lambda *a: (_ for _ in ()).throw(_NoLaunch()))
    seqlens = np.array([100, 300], np.int32)
    shape = mla.PrefillShape(2, 400, 4, 192, 128, 1 + 3)
    T, Hp = 400, 4
    q = torch.zeros((T, Hp, 192), dtype=torch.bfloat16)
    cu = torch.tensor([0, 100, 400], dtype=torch.int32)
    quant = mla.prefill_alloc_quant(shape, "cpu")
    with pytest.raises((ValueError, _NoLaunch)) as e:
        mla.prefill_quantize(shape, cu, q, q, torch.zeros((T, Hp, 128), dtype=torch.bfloat16),
                             quant=quant)
    assert e.type is _NoLaunch   # consistent sizes pass the checks
    del seqlens
    with pytest.raises(ValueError, match="v"):
        mla.prefill_quantize(shape, cu, q, q, torch.zeros((T, Hp, 192), dtype=torch.bfloat16),
                             quant=quant)
    with pytest.raises(ValueError, match="cu_seqlens"):
        mla.prefill_quantize(shape, cu[:2].contiguous(), q, q,
                             torch.zeros((T, Hp, 128), dtype=torch.bfloat16), quant=quant)
    bad = mla.PrefillQuant(**{**quant.__dict__,
                              "k_scale": torch.zeros((3, Hp), dtype=torch.float32)})
    with pytest.raises(ValueError, match="k_scale"):
        mla.prefill_attn(shape, cu, bad, 0.07)

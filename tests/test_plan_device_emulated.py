"""The device-side planner (mla_decode_plan_device) run on the CPU by the
lane-fiber emulator: its plan image must equal the host planner's
(mla_decode_plan_fixed) word for word, and lengths the host planner rejects
must give an empty plan and MLA_ERR_BAD_SHAPE.
"""
import os

import numpy as np
import pytest

import mla_paged_decode_absorbed_amd as mla
from tests.test_kernel_emulated import _available

try:
    from tests.simt_emu import harness
except ImportError:  # pragma: no cover
    harness = None

pytestmark = pytest.mark.skipif(harness is None or not _available(),
                                reason="host clang++ not available")


def _image_words(host):
    return int(host[10]) + 4 * int(host[4])        # combine offset + entries


def _compare(B, H, qmax, kv, ql, G, phases="", causal=True, P=64):
    maxp = max(1, int((max(kv) + P - 1) // P)) if B else 1
    pages = max(1, int(sum((int(x) + P - 1) // P for x in kv)))
    shape = mla.Shape.make(batch=B, num_heads=H, max_q_len=qmax, page_size=P, num_pages=pages,
                           max_pages_per_seq=maxp, causal=causal)
    old = os.environ.get("MLA_PHASES")
    os.environ["MLA_PHASES"] = phases
    try:
        host = mla.plan(shape, np.asarray(kv, np.int32),
                        None if ql is None else np.asarray(ql, np.int32), num_workgroups=G,
                        upload=False, fixed=True)
    finally:
        if old is None:
            del os.environ["MLA_PHASES"]
        else:
            os.environ["MLA_PHASES"] = old
    st, pst, img = harness.run_plan_device(B, H, qmax, P, pages, maxp, causal, kv, ql, G,
                                           env_extra={"MLA_PHASES": phases})
    assert (st, pst) == (0, 0)
    n = _image_words(host.host)
    assert np.array_equal(img[:n], host.host[:n])
    return host


@pytest.mark.parametrize("seed,B,H,qmax,G,phases", [
    (0, 64, 128, 1, 256, ""), (1, 128, 128, 2, 256, ""), (2, 16, 128, 1, 256, ""),
    (3, 7, 128, 2, 64, "2"), (4, 300, 128, 1, 256, "4"), (5, 3, 16, 8, 256, ""),
    (6, 1, 128, 1, 256, ""), (7, 40, 64, 2, 96, "4"), (8, 256, 128, 2, 256, ""),
    (9, 0, 128, 1, 256, ""), (10, 256, 128, 8, 256, ""),
])
def test_device_plan_equals_host_plan(seed, B, H, qmax, G, phases):
    rng = np.random.default_rng(seed)
    kv = rng.integers(1, int(rng.choice([100, 5000, 40000])), size=B, endpoint=True)
    ql = rng.integers(0, qmax, size=B, endpoint=True)
    kv = np.maximum(kv, ql).astype(np.int32)
    _compare(B, H, qmax, kv, ql.astype(np.int32), G, phases)


def test_device_plan_without_q_lens_and_non_causal():
    kv = np.array([0, 5, 700, 64], np.int32)
    _compare(4, 128, 2, kv, None, 32, causal=False)


@pytest.mark.parametrize("kv,ql", [
    ([100, 3000], [3, 1]),          # q_len above max_q_len
    ([1, 3000], [2, 1]),            # causal kv_len below q_len
    ([-1, 3000], [1, 1]),           # negative length
    ([100, 5000], [1, 1]),          # past the block table (4096 keys)
])
def test_device_plan_rejects_bad_lengths(kv, ql):
    st, pst, img = harness.run_plan_device(2, 128, 2, 64, 200, 64, True, np.array(kv, np.int32),
                                           np.array(ql, np.int32), 16)
    assert st == 0 and pst == int(2)                  # MLA_ERR_BAD_SHAPE
    assert img[0] == 0x504C414D and img[2] == 16      # a plan for all 16 workgroups
    assert img[3] == 0 and img[4] == 0 and img[5] == 0  # with no items, entries or partials
    ws = img[int(img[8]):int(img[8]) + 17]
    assert np.all(ws == 0)


def test_device_plan_refuses_shapes_beyond_its_lds():
    # 512 sequences x 8 tokens x 128 heads: 4096 units do not fit
    st, _, _ = harness.run_plan_device(512, 128, 8, 64, 8192, 16, True,
                                       np.full(512, 100, np.int32), np.full(512, 8, np.int32), 256)
    assert st == 3                                     # MLA_ERR_UNSUPPORTED

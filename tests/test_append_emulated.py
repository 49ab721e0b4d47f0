"""The cache-append kernel (``mla_kv_append``) run on the CPU by the lane-fiber
emulator under AddressSanitizer, against the oracle, bit for bit: every byte
of the cache and every scale, written or not, must equal the oracle's.
"""
import numpy as np
import pytest

from oracle import append_ref
from tests.append_cases import make_append_case
from tests.test_kernel_emulated import _available

try:
    from tests.simt_emu import harness
except ImportError:  # pragma: no cover
    harness = None

pytestmark = pytest.mark.skipif(harness is None or not _available(),
                                reason="host clang++ not available")


def _compare(c, new_lens="given", with_counter=True):
    nl = c["new_lens"] if new_lens == "given" else None
    want_kv, want_sc, want_sk = append_ref.kv_append_ref(
        c["kv"], c["kv_scale"], c["block_table"], c["kv_lens"], nl, c["new_rows_bits"],
        c["page_size"], c["kv_dtype"])
    got_kv, got_sc, got_sk = harness.run_append(
        c["kv"], c["kv_scale"], c["block_table"], c["kv_lens"], nl, c["new_rows_bits"],
        c["page_size"], c["kv_dtype"], with_counter=with_counter)
    assert np.array_equal(got_kv, want_kv)
    if c["kv_dtype"] == "fp8_e4m3":
        assert np.array_equal(got_sc.view(np.uint32), want_sc.view(np.uint32))
    if with_counter:
        assert got_sk == want_sk
    return want_sk


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8_e4m3"])
@pytest.mark.parametrize("P", [16, 64])
def test_decode_step_append(kv_dtype, P):
    if kv_dtype == "fp8_e4m3" and P < 64:
        pytest.skip("e4m3 caches take pages of 64 tokens or more")
    c = make_append_case([70, 5, 129, 64, 3, 1, 200], [2, 5, 1, 0, 3, 1, 8], P, kv_dtype, seed=3)
    assert _compare(c) == 0


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8_e4m3"])
def test_rows_outside_the_pool_are_skipped(kv_dtype):
    c = make_append_case([70, 5, 129, 64, 3], [2, 5, 1, 2, 3], 64, kv_dtype, seed=4)
    bt = c["block_table"]
    bt[0, 69 // 64] = -1                      # removed page
    bt[2, 128 // 64] = c["kv"].shape[0]       # page id past the pool
    c["kv_lens"][4] = 1                       # 3 new tokens at positions -2, -1, 0
    c["new_lens"][3] = 9                      # more than max_new
    assert _compare(c) == 2 + 1 + 2 + c["new_rows_bits"].shape[1]


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8_e4m3"])
def test_without_lengths_or_counter(kv_dtype):
    c = make_append_case([70, 130, 64], [4, 4, 4], 64, kv_dtype, seed=5)
    _compare(c, new_lens=None, with_counter=False)


def test_prompt_sized_append_strides_the_grid():
    # 3 x 2743 rows: more than the 2048 workgroups x 4 rows of one grid pass
    c = make_append_case([2743, 2800, 2743], [2743, 2743, 2000], 64, "bf16", seed=6,
                         max_new=2743)
    assert _compare(c) == 0


def test_prompt_sized_e4m3_append():
    c = make_append_case([900, 1000], [900, 333], 128, "fp8_e4m3", seed=7, max_new=900)
    assert _compare(c) == 0


def test_fast_paths_match_plain_arithmetic_exhaustively():
    # the kernel's reciprocal + correction quotient over every pair of bf16
    # values (|x| <= max|x|, scale >= 2^-64) against true division, and the
    # emulator's e4m3 conversion model against a plain encoder
    import os
    import subprocess
    from tests.simt_emu import build as _b
    binary = _b.build_exhaustive()
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0")
    res = subprocess.run([binary], capture_output=True, text=True, timeout=600, env=env)
    assert res.returncode == 0, res.stdout + res.stderr[-2000:]
    assert "0 differ" in res.stdout and "0 codes differ" in res.stdout

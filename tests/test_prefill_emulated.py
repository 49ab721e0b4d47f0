"""Quantized prefill on the CPU emulator (mla_prefill_quantize +
mla_prefill_attn under AddressSanitizer): codes and scales bit-exact against
the oracle's quantizers, O and LSE against the oracle's blocked softmax."""
import pytest

from oracle import prefill_ref
from tests.prefill_cases import check_attention, check_quantized
from tests.test_kernel_emulated import _available
from workloads.prefill import make_prefill_case

try:
    from tests.simt_emu import harness
except ImportError:  # pragma: no cover
    harness = None

pytestmark = pytest.mark.skipif(harness is None or not _available(),
                                reason="host clang++ not available")


def _run(case):
    nb = prefill_ref.num_blocks(case.seqlens)
    got = harness.run_prefill(case, nb)
    quant = check_quantized(case, got)
    check_attention(case, got["o"], got["lse"], quantized=quant)
    return got


def test_prefill_ragged_sequences():
    # several key blocks, a diagonal block with a ragged tail, a 1-token and
    # a 5-token sequence
    _run(make_prefill_case(seqlens=[300, 1, 5, 129], num_heads=2, seed=71))


def test_prefill_zero_rows_and_channel_offset():
    case = make_prefill_case(seqlens=[140, 60], num_heads=3, seed=72, k_bias=2.0, v_std=0.01)
    case.q[7] = 0                        # zero query rows: uniform weights
    case.k[150, 1] = 0                   # an all-zero key row: scale 1
    case.v[10:20, 2, 3] = 0              # a channel zero in part of a block
    _run(case)


def test_prefill_empty_sequence_is_skipped():
    case = make_prefill_case(seqlens=[3, 0, 130], num_heads=1, seed=73)
    got = _run(case)
    assert got["vc"].shape[0] == 3

"""The emulated kernels and the host library under UndefinedBehaviorSanitizer
as well as AddressSanitizer: integer overflow, shifts of negative values or
past the width, misaligned vector accesses and the like, anywhere in the
kernels' index arithmetic (run on the CPU by the lane-fiber emulator), the
planner or the C-ABI layer, stop the run.

A selection of the emulated suites runs against that build (EMU_BINARY names
it to the harness): every decode kernel under random schedules in both
copy-landing modes, a cache append, tree drafts, the device planner, the
input check and the quantized prefill.
The whole emulated suite passed against it in a one-off run."""
import os
import subprocess
import sys

import pytest

from tests.test_kernel_emulated import _available

pytestmark = pytest.mark.skipif(not _available(), reason="host clang++ not available")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SELECTION = [
    "tests/test_kernel_emulated.py::test_random_schedules_every_decode_kernel",
    "tests/test_append_emulated.py::test_decode_step_append",
    "tests/test_tree_emulated.py::test_tree_drafts_through_the_split_decode_kernel",
    "tests/test_plan_device_emulated.py::test_device_plan_without_q_lens_and_non_causal",
    "tests/test_check_emulated.py::test_block_table_entry_outside_the_pool",
    "tests/test_prefill_emulated.py::test_prefill_ragged_sequences",
]


def test_emulated_suites_under_ubsan():
    from tests.simt_emu import build as _b
    binary = _b.fresh_build("ubsan", ubsan=True)
    env = dict(os.environ, EMU_BINARY=binary, UBSAN_OPTIONS="print_stacktrace=1")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                          *SELECTION], env=env, cwd=ROOT, capture_output=True, text=True,
                         timeout=1500)
    assert res.returncode == 0, (res.stdout[-4000:], res.stderr[-2000:])
    assert " passed" in res.stdout and "failed" not in res.stdout

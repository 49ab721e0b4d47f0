"""bench.py's Python paths on the CPU, with the GPU stubbed out
(tests/bench_stub_run.py): every mode prints exactly one JSON line with the
fields the bench contract asks for.  The numbers are meaningless here; a mode
that raises, or a line that lacks a field, would cost a round's bench record."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
RUNNER = os.path.join(ROOT, "tests", "bench_stub_run.py")
LIB = os.path.join(ROOT, "mla_paged_decode_absorbed_amd", "libmla_decode.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="library not built")

CONTRACT = ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
            "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config")
ROOFLINE = ("bound", "achieved", "peak", "unit", "frac", "traffic")


def _launch(args):
    env = dict(os.environ)
    env.pop("MLA_DECODE_KERNEL", None)
    return subprocess.run([sys.executable, RUNNER, "--steps", "2", "--warmup", "1", *args],
                          capture_output=True, text=True, timeout=600, env=env, cwd=ROOT)


def _line(res):
    assert res.returncode == 0, res.stderr[-3000:]
    lines = [l for l in res.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, res.stdout[-2000:]
    line = json.loads(lines[0])
    for k in CONTRACT:
        assert k in line, k
    assert line["n_gpus"] == 1 and line["steps"] == 2 and line["warmup"] == 1
    assert line["data"] == "synthetic" and "workload" in line["config"]
    for k in ROOFLINE:
        assert k in line["roofline"], k
    assert line["roofline"]["bound"] in ("hbm", "mfma", "alu")
    return line


DECODE_MODES = [
    (("--graph",), "mla_decode_kernel_pairs"),
    (("--decode-kernel", "w8"), "mla_decode_kernel_w8"),
    (("--workload", "long_ctx_fp8", "--decode-kernel", "w8"), "mla_decode_kernel_w8"),
    (("--workload", "long_ctx_fp8", "--decode-kernel", "qres"), "mla_decode_kernel_qres"),
    (("--decode-kernel", "split"), "mla_decode_kernel_split"),
    (("--workload", "long_ctx_fp8", "--decode-kernel", "split"), "mla_decode_kernel_split"),
    (("--workload", "mtp_verify_bf16", "--num-workgroups", "128"), "mla_decode_kernel_pairs"),
    (("--workload", "tree_verify_bf16",), None),
]
OTHER = ["append_prompt_fp8", "sage_prefill_mix"]


@pytest.fixture(scope="module")
def runs():
    """Every mode's bench run, four processes at a time."""
    from concurrent.futures import ThreadPoolExecutor
    jobs = {"default": ("--cpu-seconds", "0.5")}
    for args, _k in DECODE_MODES:
        jobs[args] = ("--no-cpu-baseline", *args)
    for w in OTHER:
        jobs[w] = ("--no-cpu-baseline", "--workload", w)
    with ThreadPoolExecutor(max_workers=4) as ex:
        futs = {k: ex.submit(_launch, v) for k, v in jobs.items()}
        return {k: f.result() for k, f in futs.items()}


def test_default_line_with_the_oracle_baseline(runs):
    line = _line(runs["default"])
    assert line["config"]["workload"] == "v3_decode_bf16"
    cb = line["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["cores"] >= 1 and cb["value"] > 0


@pytest.mark.parametrize("args,kernel", DECODE_MODES)
def test_decode_modes(runs, args, kernel):
    line = _line(runs[args])
    if kernel:
        assert line["roofline"]["kernel"] == kernel
    assert line["cpu_baseline"] is None


@pytest.mark.parametrize("workload", OTHER)
def test_other_workloads(runs, workload):
    line = _line(runs[workload])
    assert line["config"]["workload"] == workload


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, RUNNER, "--gpus", "2"], capture_output=True,
                         text=True, timeout=600, cwd=ROOT)
    assert res.returncode != 0 and "one GPU" in res.stderr

"""The GPU test modules import and collect on the CPU: with torch.cuda
stubbed as available (tests/bench_stub_run.py), ``pytest --collect-only -m
gpu`` imports every test_gpu_* module past its GPU guard, resolves their
imports and expands their parameters, so a broken import or parametrization
shows here rather than in a GPU run.  Nothing is run."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SCRIPT = """
import sys
sys.path.insert(0, {root!r})
sys.path.insert(0, {tests!r})
import bench_stub_run
bench_stub_run.install()
import pytest
sys.exit(pytest.main(["--collect-only", "-q", "-m", "gpu", "-p", "no:cacheprovider", {tests!r}]))
"""


def test_gpu_test_modules_collect():
    code = SCRIPT.format(root=ROOT, tests=os.path.join(ROOT, "tests"))
    env = dict(os.environ, MLA_RUN_UNVALIDATED="1")
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                         timeout=600, cwd=ROOT, env=env)
    assert res.returncode == 0, (res.stdout[-3000:], res.stderr[-3000:])
    collected = [l for l in res.stdout.splitlines() if "::" in l]
    modules = {l.split("::")[0] for l in collected}
    gpu_modules = {f"tests/{f}" for f in os.listdir(os.path.join(ROOT, "tests"))
                   if f.startswith("test_gpu") and f.endswith(".py")}
    assert gpu_modules <= modules, sorted(gpu_modules - modules)
    assert len(collected) > 100

"""The GPU test modules import and collect on the CPU: with torch.cuda
stubbed as available (tests/bench_stub_run.py), ``pytest --collect-only -m
gpu`` imports every test_gpu_* module past its GPU guard, resolves their
imports and expands their parameters, so a broken import or parametrization
shows here rather than in a GPU run.  The second check collects in a copy of
the tree without the paths .gpurunignore lists (the CPU emulator among
them), which is the tree a GPU run receives.  Nothing is run."""
import fnmatch
import os
import shutil
import subprocess
import sys
import tempfile

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


def _ignored(patterns, rel):
    """tar's exclude patterns as .gpurunignore uses them: "./x" names a path
    from the top, any other pattern matches a name at any depth."""
    for p in patterns:
        if p.startswith("./"):
            if rel == p[2:] or rel.startswith(p[2:] + "/"):
                return True
        elif any(fnmatch.fnmatch(part, p) for part in rel.split("/")):
            return True
    return False


def test_gpu_test_modules_collect_in_the_uploaded_tree():
    patterns = [l.strip() for l in open(os.path.join(ROOT, ".gpurunignore"))
                if l.strip() and not l.startswith("#")]
    patterns += [".git", "gpurun_out", "__pycache__", "_build", ".pytest_cache"]
    with tempfile.TemporaryDirectory() as d:
        dst = os.path.join(d, "repo")

        def ignore(src, names):
            rel = os.path.relpath(src, ROOT)
            rel = "" if rel == "." else rel + "/"
            return [n for n in names if _ignored(patterns, rel + n)]

        shutil.copytree(ROOT, dst, ignore=ignore, symlinks=True)
        assert not os.path.exists(os.path.join(dst, "tests", "simt_emu"))
        code = SCRIPT.format(root=dst, tests=os.path.join(dst, "tests"))
        env = dict(os.environ, MLA_RUN_UNVALIDATED="1")
        res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                             timeout=600, cwd=dst, env=env)
        assert res.returncode == 0, (res.stdout[-3000:], res.stderr[-3000:])
        modules = {l.split("::")[0] for l in res.stdout.splitlines() if "::" in l}
        gpu_modules = {f"tests/{f}" for f in os.listdir(os.path.join(dst, "tests"))
                       if f.startswith("test_gpu") and f.endswith(".py")}
        assert gpu_modules <= modules, sorted(gpu_modules - modules)

"""bench.py's command line on the CPU: the one-GPU contract and the help text
(no GPU work; both paths return before torch is imported)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    for n in ("2", "8"):
        r = _run("--gpus", n)
        assert r.returncode == 2
        assert "one GPU only" in r.stderr and f"--gpus {n}" in r.stderr
        assert r.stdout == ""  # no JSON line


def test_help_lists_the_workloads():
    r = _run("--help")
    assert r.returncode == 0
    for w in ("prefill-8k-bf16-hbm", "prefill-16k-fp8-hbm", "prefill-8k-bf16-host", "decode-256",
              "spec-decode-256x4", "select-rows-8k"):
        assert w in r.stdout

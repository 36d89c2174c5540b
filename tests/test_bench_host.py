"""bench.py's command line on the host: the runs it refuses before touching a GPU."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT, capture_output=True,
                          text=True, timeout=300)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_unknown_workload_is_refused():
    r = _run("--only", "moe_backward,no_such_workload")
    assert r.returncode == 2
    assert "no_such_workload" in r.stderr
    assert r.stdout == ""

"""bench.py's command line, without a GPU: more than one GPU is refused with a message, and an
unknown workload name is rejected by the argument parser."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_unknown_workload_is_rejected():
    r = _run("--workload", "no_such_workload")
    assert r.returncode == 2
    assert "invalid choice" in r.stderr

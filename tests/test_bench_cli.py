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


def test_cpu_baseline_pool_reports_its_host():
    """The oracle baseline's process pool on a small workload: fields and a positive rate."""
    sys.path.insert(0, ROOT)
    import bench
    import workloads
    w = dict(B=1, N=256, H=3, d=64, causal=False, dtype="bf16", seed=1)
    x = workloads.make_inputs(1, 256, 3, 64, "bf16", 1, with_do=True)
    rec = bench.cpu_baseline(x, w, 2, ["attn_fwd_bf16", "attn_bwd_bf16", "attn_fwd_fp8"], 5)
    assert rec["kind"] == "oracle" and rec["value"] > 0 and rec["cores"] == 2
    assert rec["nproc"] >= 1 and rec["cpu_model"] and "2 of 3 heads" in rec["sample"]

"""Host-side parts of bench.py that need no GPU: the CPU-baseline leg (the oracle timed over a
bounded sample) and the refusal of more than one GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_cpu_baseline_record():
    import bench
    from fourier_domain_linear_amd.workloads import BY_NAME, workload_inputs

    w = BY_NAME["p4_c16_n64_f32"]
    x, W, b = workload_inputs(w, seed=0)
    r = bench.cpu_baseline(w, x, W, b, budget_s=0.2)
    assert r["kind"] == "oracle" and r["unit"] == "tokens/s"
    assert r["value"] > 0 and r["cores"] >= 1 and r["sample"]
    assert r["single_thread"]["value"] > 0
    assert isinstance(r["cpu_model"], str) and r["cpu_model"]


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""

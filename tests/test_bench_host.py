"""Host-side behaviour of bench.py that needs no GPU: more than one GPU is
refused with a message, and the CPU-oracle baselines report what they ran."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_cpu_baselines_report_their_sample():
    import bench

    one = bench.cpu_baseline(0, 1, seed=7, n_seqs_sample=1, one_core=True)
    assert one["kind"] == "oracle" and one["cores"] == 1 and one["value"] > 0
    assert one["unit"] == "window tokens/s" and "1 sequences x 1 of 1 layers" in one["sample"]
    full = bench.cpu_baseline(0, 1, seed=7, n_seqs_sample=1)
    assert full["kind"] == "oracle" and full["cores"] >= 1 and full["value"] > 0

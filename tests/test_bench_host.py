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
    import numpy as np

    import bench
    from decode_kv_cache_kara_amd import synth
    from oracle import kara_oracle as ko

    wl = synth.make_workload(0, device="cpu")
    one = bench.cpu_baseline(wl, [0], [0], one_core=True)
    assert one["kind"] == "oracle" and one["cores"] == 1 and one["value"] > 0
    assert one["unit"] == "window tokens/s" and "1 (sequence, layer) pairs" in one["sample"]
    assert one["host_cores"] >= 1
    # with outputs equal to the oracle's own, the sampled parity is all exact
    res = ko.compress(wl.q_window.double().numpy(), wl.pool.double().numpy(), wl.table.long().numpy(),
                      wl.lens.long().numpy(), wl.window, wl.protect, wl.top_k, wl.budget, wl.block_size,
                      wl.free_ids, units=[(0, 0)])
    gpu = {"scores": res["scores"].reshape(wl.n_units, -1).astype(np.float32),
           "cand": res["cand"].reshape(wl.n_units, -1), "kept": res["retained"].reshape(wl.n_units, -1)}
    full = bench.cpu_baseline(wl, [0], [0], gpu=gpu)
    assert full["kind"] == "oracle" and full["cores"] >= 1 and full["value"] > 0
    assert full["parity"]["exact"] == wl.n_units and full["parity"]["fail"] == 0


def test_spread_keeps_the_ends():
    import bench

    assert bench.spread(128, 4) == [0, 42, 85, 127]
    assert bench.spread(3, 8) == [0, 1, 2]

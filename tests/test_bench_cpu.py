"""Host-side checks of bench.py's contract (no GPU needed).

* more than one GPU is refused with a message (this library has no multi-GPU path);
* without a GPU the run fails loudly instead of measuring anything on the CPU;
* the CPU baseline (the oracle on a bounded sample) reports the fields the result line carries.
"""
import os
import subprocess
import sys

import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + list(args), cwd=ROOT,
                          capture_output=True, text=True, timeout=600)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_no_gpu_fails_loudly():
    if torch.cuda.is_available():
        return
    r = _run("--only-step")
    assert r.returncode != 0
    assert r.stdout.strip() == ""  # no result line


def test_cpu_baseline_fields():
    sys.path.insert(0, ROOT)
    import bench

    b = bench.cpu_baseline(rows=2, reps=1)
    assert b["kind"] == "oracle" and b["unit"] == "TFLOP/s" and b["value"] > 0
    assert b["cores"] >= 1 and b["os_cpu_count"] >= 1
    for key in ("sample", "cpu_model", "affinity_cpus", "cores_note"):
        assert key in b

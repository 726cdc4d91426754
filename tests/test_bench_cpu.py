"""CPU tests of bench.py's host-side pieces: the CPU-baseline leg and the refusal of more
than one GPU (no GPU is touched)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from lossless_speculative_verification_amd import workload as W  # noqa: E402


def test_cpu_baseline_is_bounded_and_complete():
    wl = W.WORKLOADS["tiny_fp32"]
    r = bench.cpu_baseline(wl, W.make_weights(wl), W.make_hidden(wl), lambda y: W.make_drafts(wl, y),
                           min_seconds=0.2, max_passes=3)
    assert set(r) == {"value", "unit", "cores", "kind", "sample"}
    assert r["kind"] == "oracle" and r["unit"] == "verified tokens/s" and r["cores"] >= 1
    assert r["value"] > 0
    passes = int(r["sample"].split()[0])
    assert 1 <= passes <= 3


def test_bench_refuses_more_than_one_gpu():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert p.returncode == 2
    assert "one GPU" in p.stderr

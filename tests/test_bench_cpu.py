"""Host-side parts of bench.py (CPU only): pair counting, the committed HBM-traffic summary,
and the one-GPU contract."""
import os
import subprocess
import sys

import pytest

import bench
from workloads import visible_pairs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_visible_pairs_match_workloads():
    for T in (1, 7, 128, 1000):
        for causal in (True, False):
            for W in (0, 1, 5, 100, 2000):
                assert bench.visible_pairs(T, causal, W) == visible_pairs(T, causal, W)


def test_traffic_summary_parses_and_covers_compulsory_bytes():
    with open(bench.TRAFFIC_FILE) as fh:
        lines = [ln.split() for ln in fh if ln.strip().startswith("traffic kernel=")]
    kinds = {dict(p.split("=", 1) for p in parts[1:])["kernel"] for parts in lines}
    assert kinds == {"fwd", "bwd_dq_dvec", "bwd_dkdv"}
    t = bench.measured_traffic("bwd_dkdv")
    if t is None:
        pytest.skip("kernel sources changed since the committed counters were taken")
    # compulsory bytes of the dK/dV pass at B=4 H=32 HKV=8 T=4096 D=128: Q, dO (bf16), K, V
    # (bf16), L, D (fp32) read once, dK, dV (fp32) written once
    B, T, H, HKV, D = 4, 4096, 32, 8, 128
    compulsory = 2 * B * T * H * D * 2 + 2 * B * T * HKV * D * 2 + 2 * B * H * T * 4 + 2 * B * T * HKV * D * 4
    assert t >= compulsory


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr

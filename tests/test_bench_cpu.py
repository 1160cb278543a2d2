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


def test_json_line_from_synthetic_timings():
    """The line's contract from made-up timings: every required key, value = the metric's
    fwd+bwd FLOPs per step time, the dominant kernel's roofline with the probe's fraction, the
    traffic lookup only for the headline workload."""
    from workloads import get_config, fwd_flops, bwd_flops
    cfg = get_config("C4")
    r = {"ms_per_step": 2.0, "ms_per_step_with_events": 2.02, "fwd_ms": 0.5, "bwd_ms": 1.5, "fwd_ms_mean": 0.51, "bwd_ms_mean": 1.52,
         "kernels_ms": {"fwd": 0.5, "bwd_dq_dvec": 0.7, "bwd_dkdv": 0.8},
         "kernels_ms_mean": {"fwd": 0.5, "bwd_dq_dvec": 0.7, "bwd_dkdv": 0.8}}
    probe = {"unit": "TFLOP/s", "normal": 1500.0, "uniform01": 1600.0, "constant": 1900.0}
    asked = []
    line = bench.make_line(cfg, r, 20, 5, 0.2, lambda k: asked.append(k) or 123, probe,
                           {"C3": {"ms_per_step": 0.35}})
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "ms_per_step_with_events", "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "kernels", "fwd_frac_peak", "fwd_bwd_frac_peak", "workloads",
                "mfma_probe"):
        assert key in line, key
    assert line["n_gpus"] == 1 and line["steps"] == 20 and line["warmup"] == 5
    assert line["dtype"] == "bf16" and line["vs_baseline"] is None and line["higher_is_better"]
    assert line["config"]["workload"] == cfg.describe() and line["config"]["T"] == 4096
    want = (fwd_flops(cfg) + bwd_flops(cfg)) / 2.0e-3 / 1e12
    assert abs(line["value"] - want) < 0.01
    roof = line["roofline"]
    assert roof["kernel"] == "bwd_dkdv" and roof["bound"] == "mfma" and roof["peak"] == bench.PEAK_BF16
    work = 8.0 * cfg.D * cfg.B * cfg.H * bench.visible_pairs(cfg.T, cfg.causal, cfg.window)
    assert abs(roof["achieved"] - work / 0.8e-3 / 1e12) < 0.1
    assert abs(roof["frac"] - roof["achieved"] / bench.PEAK_BF16) < 1e-3
    assert abs(roof["frac_measured_peak"] - roof["achieved"] / 1500.0) < 1e-3
    assert roof["traffic"] == 123 and asked == ["bwd_dkdv"]
    # another workload: no traffic lookup
    other = bench.make_line(get_config("C3"), r, 20, 5, 0.2, lambda k: 1 / 0)
    assert other["roofline"]["traffic"] is None

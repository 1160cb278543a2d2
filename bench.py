"""Benchmark of the fused attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config C4] [--no-cpu-baseline]
                    [--no-extra-workloads] [--no-mfma-probe] [--prologue] [--calibrate-copy]

A step is one pass of the whole path over one batch of synthetic input already resident in
HBM: flash_attn_fwd, then flash_attn_bwd (the public entry points; the backward includes its
stream-ordered Dvec workspace).  W untimed steps, then exactly K timed steps between device
synchronisations give `ms_per_step` and `value`.  A second run of K steps with HIP events
recorded on the launch stream around each call gives the per-call medians `fwd_ms` and
`bwd_ms` (and `ms_per_step_with_events`, its wall time per step).  A third run of K steps
calls the three kernels through their stage entry points (flash_attn_fwd,
flash_attn_bwd_dq_dvec, flash_attn_bwd_dkdv, the kernels flash_attn_bwd runs) with events
between them, for the per-kernel medians in `kernels` and the dominant kernel's `roofline`.
Prints one JSON line.

FLOP convention: forward 4*B*H*T^2*D (halved when causal), backward 2.5x that; the metric is
fwd+bwd TFLOP/s, with the forward alone and the fraction of the MI355X dense bf16 MFMA peak
(2516.6 TFLOP/s = 256 CU x 2.4 GHz x 4096 FLOP/clk) reported beside it.  Per kernel, the
algorithmic work is FLOP per visible (query, key) pair times the visible pairs.

`workloads` carries the same figures for the other bf16 workloads (D=64 MHA and the sliding
window; the window one also counted by its visible pairs) unless --no-extra-workloads.

`roofline.measured_peak` is the bf16 MFMA rate the chip sustains in the library's MFMA probe
(flash_attn_mfma_rate_probe: 16x16x32 MFMAs, the shape the attention kernels use) on N(0,1)
operands, the distribution of this workload's inputs; `mfma_probe` lists it beside the rates
on uniform [0,1) and constant operands.

roofline.traffic is the HBM byte count (read + write) per launch of the dominant kernel, taken
from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE summary scaled by a plain device copy of
known size (`--calibrate-copy` adds that copy to a profiled run); it is null for other
workloads and whenever the kernel sources no longer match the ones the counters were taken on.

The CPU baseline times the fp64 oracle (a plain materialised-softmax reference) on the host
cores on a bounded sample of the same workload: whole (batch, KV-head) groups, the forward for
about a third of the budget, then forward + backward for the rest.
"""
import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16 = 2516.6    # TFLOP/s, dense bf16 MFMA (AMD MI355X specification)
PEAK_FP32 = 157.3     # TFLOP/s, fp32 matrix / vector
COPY_BYTES = 512 * 1024 * 1024
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_c4_hbm_traffic.md")
CSRC = os.path.join(ROOT, "online_softmax_fwd_flash_amd", "csrc")
METRIC = "causal attn TFLOP/s fwd & fwd+bwd (bf16, GQA, T=4096, D=128); % MFMA peak"
EXTRA_WORKLOADS = ("C3", "C5")
PROBE_GRID, PROBE_ITERS = 2048, 1000   # MFMA probe launch: grid * 4 * iters * 32 MFMAs
MFMA_FLOP = 2 * 16 * 16 * 32           # one bf16 16x16x32 MFMA


def visible_pairs(T, causal, window):
    """Exact number of (query, key) pairs kept per (batch, head)."""
    import numpy as np
    i = np.arange(T, dtype=np.int64)
    hi = i if causal else np.full(T, T - 1)
    lo = np.maximum(0, i - window + 1) if window > 0 else np.zeros(T, dtype=np.int64)
    return int(np.maximum(0, hi - lo + 1).sum())


TRAFFIC_TUS = ("fwd_b16.hip", "bwd_b16.hip")   # define the kernels the traffic lines cover


def kernel_source_hash():
    """sha256 over the sources of the measured attention kernels: their translation units and
    the csrc headers these include (transitively), sorted by name, with comments and whitespace
    removed so that edits to comments alone, or to code outside these kernels (the C ABI, the
    workspace cache), keep the hash."""
    import hashlib
    import re
    files, todo = set(), list(TRAFFIC_TUS)
    while todo:
        f = todo.pop()
        if f in files or not os.path.exists(os.path.join(CSRC, f)):
            continue
        files.add(f)
        with open(os.path.join(CSRC, f)) as fh:
            todo += re.findall(r'^\s*#include\s+"([^"]+)"', fh.read(), flags=re.M)
    h = hashlib.sha256()
    for f in sorted(files):
        with open(os.path.join(CSRC, f)) as fh:
            code = fh.read()
        code = re.sub(r"/\*.*?\*/", " ", code, flags=re.S)
        code = re.sub(r"//[^\n]*", " ", code)
        h.update(f.encode())
        h.update(" ".join(code.split()).encode())
    return h.hexdigest()


def measured_traffic(kernel):
    """HBM bytes per launch (read + write) of `kernel` on the B=4 H=32 HKV=8 T=4096 D=128 causal
    workload, from the committed counter summary; None when there is none or when the kernel
    sources changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as fh:
            lines = [ln.split() for ln in fh if ln.strip().startswith("traffic kernel=")]
    except OSError:
        return None
    sha = kernel_source_hash()
    for parts in lines:
        kv = dict(p.split("=", 1) for p in parts[1:])
        if kv.get("kernel") == kernel and kv.get("source_sha256") == sha:
            return int(kv["read_bytes"]) + int(kv["write_bytes"])
    return None


def cpu_baseline(cfg, budget_s=15.0):
    """Time the fp64 oracle on the host cores: whole (b, kv-head) groups, the forward for a
    third of the budget, then forward + backward for the rest.  BLAS runs on every core the
    process may use."""
    import contextlib
    import oracle
    from workloads import make_inputs, fwd_flops
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_limits, threadpool_info
        limits = threadpool_limits(limits=cores)
    except Exception:  # pragma: no cover - threadpoolctl missing
        threadpool_info, limits = None, contextlib.nullcontext()
    with limits:
        blas = (max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
                if threadpool_info else None)
        q, k, v, do = make_inputs(cfg)
        groups = [(b, g) for b in range(cfg.B) for g in range(cfg.HKV)]
        rep = cfg.H // cfg.HKV

        def timed(fn, budget):
            done, t0 = 0, time.perf_counter()
            for grp in groups:
                fn(grp)
                done += 1
                if time.perf_counter() - t0 >= budget:
                    break
            return done, time.perf_counter() - t0

        n_f, t_f = timed(lambda grp: oracle.attn_fwd(
            q, k, v, cfg.scale, cfg.causal, cfg.window,
            pairs=[(grp[0], h) for h in range(grp[1] * rep, (grp[1] + 1) * rep)]), budget_s / 3)
        n_fb, t_fb = timed(lambda grp: oracle.attn_bwd(
            q, k, v, do, cfg.scale, cfg.causal, cfg.window, groups=[grp]), budget_s * 2 / 3)
    per_group = fwd_flops(cfg) / (cfg.B * cfg.HKV)
    return {"value": 3.5 * per_group * n_fb / t_fb / 1e12, "unit": "TFLOP/s",
            "cores": blas or cores, "kind": "oracle",
            "fwd_value": per_group * n_f / t_f / 1e12,
            "host_cores": cores, "blas_threads": blas,
            "sample": f"{n_f} (forward) then {n_fb} (forward + backward) of the {len(groups)} "
                      f"(batch, kv-head) groups of the {cfg.describe()} workload "
                      f"({rep} query heads each) in fp64 numpy, {t_f:.1f} s + {t_fb:.1f} s wall; "
                      f"BLAS threads {blas} of {cores} usable cores"}


def time_prologue(cfg, steps, warmup):
    """flash_attn_qk_norm_rope on the workload's B*T tokens (packed QK of 2*H heads of D), the
    average of `steps` launches by HIP events on the launch stream.  Algorithmic bytes: the QK
    projection read once, Q and K written once, both factor tables read once."""
    import torch
    import online_softmax_fwd_flash_amd as fa
    from workloads import make_qk_packed, rotary_tables
    tokens, heads, D = cfg.B * cfg.T, cfg.H, cfg.D
    dev = torch.device("cuda:0")
    qk = make_qk_packed(tokens, heads, D, cfg.dtype, seed=cfg.seed).to(dev)
    f1, f2 = (t.to(dev) for t in rotary_tables(tokens, D, D))
    oq = torch.empty(tokens, heads, D, device=dev, dtype=qk.dtype)
    ok = torch.empty_like(oq)
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        fa.flash_attn_qk_norm_rope(qk, f1, f2, heads, out_q=oq, out_k=ok)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for _ in range(steps):
        fa.flash_attn_qk_norm_rope(qk, f1, f2, heads, out_q=oq, out_k=ok)
    ev[1].record(stream)
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / steps
    esz = qk.element_size()
    nbytes = 2 * tokens * 2 * heads * D * esz + 2 * tokens * D * 4
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"workload": f"qk_norm_rope {cfg.dtype} tokens={tokens} heads={heads} D={D}",
            "ms": round(ms, 4), "bound": "hbm", "bytes": nbytes, "achieved": round(gbs, 1),
            "unit": "GB/s", "peak": 8000.0, "frac": round(gbs / 8000.0, 4)}


def mfma_probe(steps=10, warmup=3):
    """bf16 MFMA rate (TFLOP/s, median of `steps` launches) of the library's probe kernel on
    three operand distributions."""
    import torch
    import online_softmax_fwd_flash_amd as fa
    dev = torch.device("cuda:0")
    g = torch.Generator("cpu").manual_seed(1234)
    dists = {
        "normal": torch.randn(4096, generator=g),
        "uniform01": torch.rand(4096, generator=g),
        "constant": torch.ones(4096),
    }
    out = torch.empty(PROBE_GRID * 256, device=dev, dtype=torch.float32)
    stream = torch.cuda.current_stream()
    flop = PROBE_GRID * 4 * PROBE_ITERS * 32 * MFMA_FLOP
    res = {}
    for name, vals in dists.items():
        ops = vals.to(torch.bfloat16).to(dev)
        for _ in range(warmup):
            fa.flash_attn_mfma_rate_probe(ops, out, PROBE_GRID, PROBE_ITERS)
        ts = []
        for _ in range(steps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fa.flash_attn_mfma_rate_probe(ops, out, PROBE_GRID, PROBE_ITERS)
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        res[name] = round(flop / (statistics.median(ts) * 1e-3) / 1e12, 1)
    return {"unit": "TFLOP/s", "kernel": "mfma_probe_kernel (bf16 16x16x32, the attention "
            "kernels' shape; 8 independent accumulators per wave)", "grid": PROBE_GRID,
            "iters": PROBE_ITERS, **res}


PREWARM_S = 0.2


def run_workload(cfg, steps, warmup, prewarm_s=PREWARM_S):
    """Time one workload: the public entry points (headline) and the stage entry points
    (per-kernel breakdown).  Before the `warmup` steps, untimed steps run for `prewarm_s`
    seconds, so the GPU's clocks have settled at this workload's load whatever ran before it.
    Returns a dict of timings in ms."""
    import torch
    import online_softmax_fwd_flash_amd as fa
    from workloads import make_inputs

    dev = torch.device("cuda:0")
    q, k, v, do = (t.to(dev) for t in make_inputs(cfg))
    B, T, H = cfg.B, cfg.T, cfg.H
    f32 = torch.float32
    o = torch.empty_like(q)
    lse = torch.empty(B, H, T, device=dev, dtype=f32)
    dvec = torch.empty(B, H, T, device=dev, dtype=f32)
    dq = torch.empty(q.shape, device=dev, dtype=f32)
    dk = torch.empty(k.shape, device=dev, dtype=f32)
    dv = torch.empty(k.shape, device=dev, dtype=f32)
    kw = dict(causal=cfg.causal, window=cfg.window, scale=cfg.scale, tiles=cfg.tiles)
    stream = torch.cuda.current_stream()

    def public(ev=None):
        if ev is not None:
            ev[0].record(stream)
        fa.flash_attn_fwd(q, k, v, out=o, lse=lse, **kw)
        if ev is not None:
            ev[1].record(stream)
        fa.flash_attn_bwd(q, k, v, o, lse, do, dq=dq, dk=dk, dv=dv, **kw)
        if ev is not None:
            ev[2].record(stream)

    def stages(ev):
        ev[0].record(stream)
        fa.flash_attn_fwd(q, k, v, out=o, lse=lse, **kw)
        ev[1].record(stream)
        fa.flash_attn_bwd_dq_dvec(q, k, v, o, do, lse, dvec=dvec, dq=dq, **kw)
        ev[2].record(stream)
        fa.flash_attn_bwd_dkdv(q, k, v, do, lse, dvec, dk=dk, dv=dv, **kw)
        ev[3].record(stream)

    def events(n):
        return [[torch.cuda.Event(enable_timing=True) for _ in range(n)] for _ in range(steps)]

    t_end = time.perf_counter() + prewarm_s
    while time.perf_counter() < t_end:
        public()
        torch.cuda.synchronize()
    for _ in range(warmup):
        public()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        public()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    ev_pub = events(3)
    t0 = time.perf_counter()
    for s in range(steps):
        public(ev_pub[s])
    torch.cuda.synchronize()
    wall_ev = time.perf_counter() - t0

    ev_st = events(4)
    for s in range(steps):
        stages(ev_st[s])
    torch.cuda.synchronize()

    def med(evs, i):
        return statistics.median(e[i].elapsed_time(e[i + 1]) for e in evs)

    def mean(evs, i):
        return sum(e[i].elapsed_time(e[i + 1]) for e in evs) / len(evs)

    out = {"ms_per_step": wall * 1e3 / steps, "ms_per_step_with_events": wall_ev * 1e3 / steps,
           "fwd_ms": med(ev_pub, 0), "bwd_ms": med(ev_pub, 1),
           "fwd_ms_mean": mean(ev_pub, 0), "bwd_ms_mean": mean(ev_pub, 1),
           "kernels_ms": {"fwd": med(ev_st, 0), "bwd_dq_dvec": med(ev_st, 1),
                          "bwd_dkdv": med(ev_st, 2)},
           "kernels_ms_mean": {"fwd": mean(ev_st, 0), "bwd_dq_dvec": mean(ev_st, 1),
                               "bwd_dkdv": mean(ev_st, 2)}}
    del q, k, v, do, o, lse, dvec, dq, dk, dv
    torch.cuda.empty_cache()
    return out


def kernel_table(cfg, kernels_ms, kernels_ms_mean, peak):
    """Per-kernel achieved TFLOP/s from algorithmic work: FLOP per visible score x visible
    scores (forward 4D: QK^T, PV; dQ pass 6D: QK^T, dO V^T, dS K; dK/dV pass 8D: QK^T, dO V^T,
    P^T dO, dS^T Q), over the average event-timed launch duration (the median beside it)."""
    vis = cfg.B * cfg.H * visible_pairs(cfg.T, cfg.causal, cfg.window)
    work = {"fwd": 4.0 * cfg.D * vis, "bwd_dq_dvec": 6.0 * cfg.D * vis,
            "bwd_dkdv": 8.0 * cfg.D * vis}
    table = {}
    for n, ms in kernels_ms.items():
        mean = kernels_ms_mean[n]
        ach = work[n] / (mean * 1e-3) / 1e12
        table[n] = {"ms": round(ms, 4), "ms_mean": round(mean, 4), "bound": "mfma",
                    "achieved": round(ach, 1), "unit": "TFLOP/s", "frac": round(ach / peak, 4),
                    "work": work[n]}
    return table, vis


def summarize(cfg, r, peak):
    """Metric figures of one workload's timings."""
    from workloads import fwd_flops, bwd_flops
    ff, bf = fwd_flops(cfg), bwd_flops(cfg)
    kernels, vis = kernel_table(cfg, r["kernels_ms"], r["kernels_ms_mean"], peak)
    s = {
        "workload": cfg.describe(),
        "ms_per_step": round(r["ms_per_step"], 4),
        "ms_per_step_with_events": round(r["ms_per_step_with_events"], 4),
        "fwd_bwd_tflops": round((ff + bf) / (r["ms_per_step"] * 1e-3) / 1e12, 2),
        "fwd_ms": round(r["fwd_ms"], 4),
        "bwd_ms": round(r["bwd_ms"], 4),
        "fwd_tflops": round(ff / (r["fwd_ms"] * 1e-3) / 1e12, 2),
        "fwd_frac_peak": round(ff / (r["fwd_ms"] * 1e-3) / 1e12 / peak, 4),
        "fwd_bwd_frac_peak": round((ff + bf) / (r["ms_per_step"] * 1e-3) / 1e12 / peak, 4),
        "kernels": kernels,
    }
    if cfg.window:
        # the metric's formula counts T^2/2 pairs per head; a window keeps far fewer, so the
        # formula's fractions of peak exceed 1 and only the window-aware ones are meaningful
        wa = 4.0 * cfg.D * vis
        fwa = wa / (r["fwd_ms"] * 1e-3) / 1e12
        fbwa = 3.5 * wa / (r["ms_per_step"] * 1e-3) / 1e12
        s["fwd_tflops_window_aware"] = round(fwa, 2)
        s["fwd_frac_peak_window_aware"] = round(fwa / peak, 4)
        s["fwd_bwd_tflops_window_aware"] = round(fbwa, 2)
        s["fwd_bwd_frac_peak_window_aware"] = round(fbwa / peak, 4)
    return s


def make_line(cfg, r, steps, warmup, prewarm, traffic, probe=None, extra=None):
    """The JSON line (without cpu_baseline / prologue) from one workload's timings `r` (as
    run_workload returns them): `traffic(kernel)` gives the committed HBM bytes per launch or
    None, `probe` the MFMA probe's rates, `extra` the other workloads' summaries."""
    from workloads import fwd_flops, bwd_flops
    peak = PEAK_BF16 if cfg.dtype == "bf16" else PEAK_FP32
    s = summarize(cfg, r, peak)
    ff, bf = fwd_flops(cfg), bwd_flops(cfg)
    value = (ff + bf) / (r["ms_per_step"] * 1e-3) / 1e12
    kernels = s["kernels"]
    dom = max(kernels, key=lambda n: kernels[n]["ms"])
    dk_ = kernels[dom]
    roofline = {"bound": dk_["bound"], "achieved": dk_["achieved"], "peak": peak,
                "unit": dk_["unit"], "frac": dk_["frac"], "kernel": dom,
                "traffic": traffic(dom) if cfg.name == "C4" else None}
    if probe is not None:
        roofline["measured_peak"] = probe["normal"]
        roofline["measured_peak_operands"] = "N(0,1) bf16 (the workload's input distribution)"
        roofline["frac_measured_peak"] = round(dk_["achieved"] / probe["normal"], 4)
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(r["ms_per_step"], 4),
        "ms_per_step_with_events": round(r["ms_per_step_with_events"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded i.i.d. N(0,1) Q, K, V, dO)",
        "config": {"workload": cfg.describe(), "B": cfg.B, "H": cfg.H, "HKV": cfg.HKV,
                   "T": cfg.T, "D": cfg.D, "causal": cfg.causal, "window": cfg.window,
                   "seed": cfg.seed},
        "fwd_tflops": s["fwd_tflops"],
        "fwd_frac_peak": s["fwd_frac_peak"],
        "fwd_bwd_frac_peak": round(value / peak, 4),
        "fwd_ms": s["fwd_ms"],
        "bwd_ms": s["bwd_ms"],
        "timing": ("each workload: untimed steps for %.1f s (clock settling), the warmup "
                   "steps, then the timed steps (no events between the calls); fwd_ms / "
                   "bwd_ms: medians of per-call HIP events on flash_attn_fwd and "
                   "flash_attn_bwd over a second run of as many steps; kernels: the stage "
                   "entry points over a third run, HIP events on the launch stream (ms: "
                   "median, ms_mean: mean; achieved = work FLOP / mean)"
                   % prewarm),
        "fwd_ms_mean": round(r["fwd_ms_mean"], 4),
        "bwd_ms_mean": round(r["bwd_ms_mean"], 4),
        "kernels": kernels,
        "roofline": roofline,
    }
    for key in ("fwd_tflops_window_aware", "fwd_frac_peak_window_aware",
                "fwd_bwd_tflops_window_aware", "fwd_bwd_frac_peak_window_aware"):
        if key in s:
            out[key] = s[key]
    if probe is not None:
        out["mfma_probe"] = probe
    if extra is not None:
        out["workloads"] = extra
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="C4")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--prewarm", type=float, default=PREWARM_S,
                    help="seconds of untimed steps before each workload's warmup steps")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--no-extra-workloads", action="store_true",
                    help="skip the D=64 MHA and sliding-window workloads")
    ap.add_argument("--no-mfma-probe", action="store_true",
                    help="skip the MFMA-rate probe (roofline.measured_peak)")
    ap.add_argument("--prologue", action="store_true",
                    help="also time the QK RMS-norm + rotary prologue on the workload's tokens "
                         "(B*T tokens, H heads, D, in the workload dtype) and report it in its "
                         "own 'prologue' object")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after timing, copy a 512 MiB device buffer once (a plain copy of known "
                         "size, for scaling hardware byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the path has no multi-GPU component); "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)

    import torch
    from workloads import get_config

    cfg = get_config(args.config)
    r = run_workload(cfg, args.steps, args.warmup, args.prewarm)

    if args.calibrate_copy:
        dev = torch.device("cuda:0")
        src = torch.empty(COPY_BYTES // 4, device=dev, dtype=torch.float32).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # the other workloads before the probe: each is timed after its own clock settling
    extra = None
    if not args.no_extra_workloads and cfg.name == "C4":
        extra = {}
        for name in EXTRA_WORKLOADS:
            c = get_config(name)
            rr = run_workload(c, args.steps, args.warmup, args.prewarm)
            extra[name] = summarize(c, rr, PEAK_BF16 if c.dtype == "bf16" else PEAK_FP32)
    probe = mfma_probe() if (not args.no_mfma_probe and cfg.dtype == "bf16") else None
    out = make_line(cfg, r, args.steps, args.warmup, args.prewarm, measured_traffic, probe,
                    extra)
    if args.prologue:
        out["prologue"] = time_prologue(cfg, args.steps, args.warmup)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

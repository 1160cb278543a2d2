"""Benchmark of the fused attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config C4] [--no-cpu-baseline]

A step is one pass of the whole path over one batch of synthetic input already resident in
HBM: forward (flash_attn_fwd) and backward (flash_attn_bwd_dq_dvec, then flash_attn_bwd_dkdv —
the two kernels flash_attn_bwd runs, called through their own entry points so each can be
timed with HIP events on the launch stream).  Prints one JSON line.

FLOP convention: forward 4*B*H*T^2*D (halved when causal), backward 2.5x that; the metric is
fwd+bwd TFLOP/s, with the forward alone and the fraction of the MI355X dense bf16 MFMA peak
(2516.6 TFLOP/s = 256 CU x 2.4 GHz x 4096 FLOP/clk) reported beside it.

roofline.traffic is the HBM byte count (read + write) per launch of the dominant kernel, taken
from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE summary scaled by a plain device copy of
known size (`--calibrate-copy` adds that copy to a profiled run); it is null for other
workloads and whenever the kernel sources no longer match the ones the counters were taken on.

The CPU baseline times the fp64 oracle (a plain materialised-softmax reference) on the host
cores on a bounded sample of the same workload: whole (batch, KV-head) groups, forward and
backward, until about 10 s have elapsed.
"""
import argparse
import json
import math
import os
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


def visible_pairs(T, causal, window):
    """Exact number of (query, key) pairs kept per (batch, head)."""
    import numpy as np
    i = np.arange(T, dtype=np.int64)
    hi = i if causal else np.full(T, T - 1)
    lo = np.maximum(0, i - window + 1) if window > 0 else np.zeros(T, dtype=np.int64)
    return int(np.maximum(0, hi - lo + 1).sum())


def kernel_source_hash():
    """sha256 over the kernel sources (csrc/*.hip and *.h, sorted by name), with comments and
    whitespace removed so that edits to comments alone keep the hash."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        if f.endswith((".hip", ".h")):
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


def cpu_baseline(cfg, budget_s=10.0):
    """Time the fp64 oracle (fwd + bwd of whole (b, kv-head) groups) on the host cores."""
    import numpy as np
    import oracle
    from workloads import make_inputs, fwd_flops
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - threadpoolctl missing
        threads = None
    q, k, v, do = make_inputs(cfg)
    groups = [(b, g) for b in range(cfg.B) for g in range(cfg.HKV)]
    done, t0 = 0, time.perf_counter()
    for grp in groups:
        oracle.attn_bwd(q, k, v, do, cfg.scale, cfg.causal, cfg.window, groups=[grp])
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    per_group = 3.5 * fwd_flops(cfg) / (cfg.B * cfg.HKV)
    cores = len(os.sched_getaffinity(0))
    return {"value": per_group * done / dt / 1e12, "unit": "TFLOP/s", "cores": threads or cores,
            "kind": "oracle",
            "sample": f"{done} of {len(groups)} (batch, kv-head) groups of the "
                      f"{cfg.describe()} workload "
                      f"({cfg.H // cfg.HKV} query heads each), fwd+bwd in fp64 numpy, "
                      f"{dt:.1f} s wall; host has {cores} usable cores"}


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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="C4")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
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
    import online_softmax_fwd_flash_amd as fa
    from workloads import get_config, make_inputs, fwd_flops, bwd_flops

    cfg = get_config(args.config)
    dev = torch.device("cuda:0")
    q, k, v, do = (t.to(dev) for t in make_inputs(cfg))
    B, T, H, HKV, D = cfg.B, cfg.T, cfg.H, cfg.HKV, cfg.D
    f32 = torch.float32
    o = torch.empty_like(q)
    lse = torch.empty(B, H, T, device=dev, dtype=f32)
    dvec = torch.empty(B, H, T, device=dev, dtype=f32)
    dq = torch.empty(q.shape, device=dev, dtype=f32)
    dk = torch.empty(k.shape, device=dev, dtype=f32)
    dv = torch.empty(k.shape, device=dev, dtype=f32)
    kw = dict(causal=cfg.causal, window=cfg.window, scale=cfg.scale, tiles=cfg.tiles)
    stream = torch.cuda.current_stream()
    names = ["fwd", "bwd_dq_dvec", "bwd_dkdv"]

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        fa.flash_attn_fwd(q, k, v, out=o, lse=lse, **kw)
        if ev is not None:
            ev[1].record(stream)
        fa.flash_attn_bwd_dq_dvec(q, k, v, o, do, lse, dvec=dvec, dq=dq, **kw)
        if ev is not None:
            ev[2].record(stream)
        fa.flash_attn_bwd_dkdv(q, k, v, do, lse, dvec, dk=dk, dv=dv, **kw)
        if ev is not None:
            ev[3].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
              for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(events[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_kernel = {n: 0.0 for n in names}
    for ev in events:
        for i, n in enumerate(names):
            per_kernel[n] += ev[i].elapsed_time(ev[i + 1])
    per_kernel = {n: t / args.steps for n, t in per_kernel.items()}   # ms per launch

    if args.calibrate_copy:
        src = torch.empty(COPY_BYTES // 4, device=dev, dtype=torch.float32).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    ms_step = wall * 1e3 / args.steps
    ff, bf = fwd_flops(cfg), bwd_flops(cfg)
    fwd_ms = per_kernel["fwd"]
    bwd_ms = per_kernel["bwd_dq_dvec"] + per_kernel["bwd_dkdv"]
    value = (ff + bf) / (ms_step * 1e-3) / 1e12
    peak = PEAK_BF16 if cfg.dtype == "bf16" else PEAK_FP32

    # algorithmic work per launch: FLOP per visible score x visible scores
    vis = B * H * visible_pairs(T, cfg.causal, cfg.window)
    algo = {
        "fwd": ("mfma", 4.0 * D * vis),                    # Q K^T and P V
        "bwd_dkdv": ("mfma", 8.0 * D * vis),               # Q K^T, dO V^T, P^T dO, dS^T Q
        "bwd_dq_dvec": ("mfma", 6.0 * D * vis),            # Q K^T, dO V^T, dS K (+ rowsum(dO O))
    }
    kernels = {}
    for n in names:
        bound, work = algo[n]
        ach = work / (per_kernel[n] * 1e-3) / 1e12
        kernels[n] = {"ms": round(per_kernel[n], 4), "bound": bound, "achieved": round(ach, 1),
                      "unit": "TFLOP/s", "frac": round(ach / peak, 4)}
    dom = max(names, key=lambda n: per_kernel[n])
    dk_ = kernels[dom]
    roofline = {"bound": dk_["bound"], "achieved": dk_["achieved"],
                "peak": peak, "unit": dk_["unit"],
                "frac": dk_["frac"], "kernel": dom,
                "traffic": measured_traffic(dom) if cfg.name == "C4" else None}

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded i.i.d. N(0,1) Q, K, V, dO)",
        "config": {"workload": cfg.describe(), "B": B, "H": H, "HKV": HKV, "T": T, "D": D,
                   "causal": cfg.causal, "window": cfg.window, "seed": cfg.seed},
        "fwd_tflops": round(ff / (fwd_ms * 1e-3) / 1e12, 2),
        "fwd_frac_peak": round(ff / (fwd_ms * 1e-3) / 1e12 / peak, 4),
        "fwd_bwd_tflops_events": round((ff + bf) / ((fwd_ms + bwd_ms) * 1e-3) / 1e12, 2),
        "fwd_bwd_frac_peak": round(value / peak, 4),
        "fwd_ms": round(fwd_ms, 4),
        "bwd_ms": round(bwd_ms, 4),
        "kernels": kernels,
        "roofline": roofline,
    }
    if cfg.window:
        # the metric's formula counts T^2/2 pairs per head; a window keeps far fewer, so the
        # formula's fractions of peak exceed 1 and only the window-aware ones are meaningful
        wa = 4.0 * D * vis
        fwa = wa / (fwd_ms * 1e-3) / 1e12
        fbwa = 3.5 * wa / (ms_step * 1e-3) / 1e12
        out["fwd_tflops_window_aware"] = round(fwa, 2)
        out["fwd_frac_peak_window_aware"] = round(fwa / peak, 4)
        out["fwd_bwd_tflops_window_aware"] = round(fbwa, 2)
        out["fwd_bwd_frac_peak_window_aware"] = round(fbwa / peak, 4)
    if args.prologue:
        out["prologue"] = time_prologue(cfg, args.steps, args.warmup)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

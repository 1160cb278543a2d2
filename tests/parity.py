"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI, run the fp64
oracle on the same seeded inputs, and compare to the tolerances of each dtype."""
import math
import sys

import numpy as np
import torch

import oracle
import online_softmax_fwd_flash_amd as fa
from workloads import make_inputs_like

# f32 path: max-abs <= 1e-4 on every output.  bf16 path (bf16 in, fp32 accumulate):
# max-abs <= 2e-2 and relative L2 <= 5e-3 per tensor, against the oracle on the same
# bf16-rounded inputs.  fp16 path: the same arithmetic with the 16-bit roundings (inputs
# aside, P and dS as MFMA operands and the stored O) at a unit roundoff of 2^-11 instead of
# 2^-8, so the bf16 bounds scaled by 2^-3, with a factor 2 of margin: max-abs <= 5e-3 and
# relative L2 <= 1.25e-3.
TOL = {"f32": dict(max_abs=1e-4, rel_l2=None), "bf16": dict(max_abs=2e-2, rel_l2=5e-3),
       "f16": dict(max_abs=5e-3, rel_l2=1.25e-3)}


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def compare(name, got, want, dtype, mask=None):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    if mask is not None:
        got, want = got[mask], want[mask]
    assert got.shape == want.shape, (name, got.shape, want.shape)
    assert np.isfinite(got).all(), f"{name}: non-finite values (unwritten or overflow)"
    err = np.abs(got - want)
    max_abs = float(err.max()) if err.size else 0.0
    rel = float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-30)) if err.size else 0.0
    tol = TOL[dtype]
    assert max_abs <= tol["max_abs"], f"{name}: max-abs {max_abs:.3e} > {tol['max_abs']}"
    # A relative bound needs a nonzero reference: a tensor that is zero up to fp64 rounding
    # (dQ and dK when every row sees a single key, e.g. T = 1) is held to max-abs alone.
    ref_rms = float(np.sqrt(np.mean(want ** 2))) if want.size else 0.0
    if tol["rel_l2"] is not None and ref_rms > 1e-9:
        assert rel <= tol["rel_l2"], f"{name}: rel-L2 {rel:.3e} > {tol['rel_l2']}"
    return max_abs, rel


def gpu_fwd(q, k, v, causal, window, scale, tiles=(0, 0)):
    dev = torch.device("cuda:0")
    qd, kd, vd = (t.to(dev).contiguous() for t in (q, k, v))
    B, T, H, D = q.shape
    o = torch.full_like(qd, float("nan"))
    lse = torch.full((B, H, T), float("nan"), device=dev, dtype=torch.float32)
    fa.flash_attn_fwd(qd, kd, vd, causal=causal, window=window, scale=scale, out=o, lse=lse,
                      tiles=tiles)
    torch.cuda.synchronize()
    return o, lse, (qd, kd, vd)


def gpu_bwd(dev_inputs, o, lse, do, causal, window, scale, tiles=(0, 0)):
    qd, kd, vd = dev_inputs
    dod = do.to(qd.device).contiguous()
    nan = float("nan")
    dq = torch.full(qd.shape, nan, device=qd.device, dtype=torch.float32)
    dk = torch.full(kd.shape, nan, device=qd.device, dtype=torch.float32)
    dv = torch.full(kd.shape, nan, device=qd.device, dtype=torch.float32)
    fa.flash_attn_bwd(qd, kd, vd, o, lse, dod, causal=causal, window=window, scale=scale,
                      dq=dq, dk=dk, dv=dv, tiles=tiles)
    torch.cuda.synchronize()
    return dq, dk, dv


def check_case(B, T, H, HKV, D, dtype, causal, window, seed, tiles=(0, 0), backward=True,
               scale=None):
    """Full comparison of every output against the oracle (small shapes)."""
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    log(f"case B={B} T={T} H={H} HKV={HKV} D={D} {dtype} causal={causal} window={window} "
        f"tiles={tiles} seed={seed}")
    q, k, v, do = make_inputs_like(B, T, H, HKV, D, dtype, seed)
    o, lse, dev = gpu_fwd(q, k, v, causal, window, scale, tiles)
    if backward:
        ref = oracle.attn_bwd(q, k, v, do, scale, causal, window)
        compare("O", to_np(o), ref["o"], dtype)
        compare("L", to_np(lse), ref["lse"], dtype)
        dq, dk, dv = gpu_bwd(dev, o, lse, do, causal, window, scale, tiles)
        compare("dQ", to_np(dq), ref["dq"], dtype)
        compare("dK", to_np(dk), ref["dk"], dtype)
        compare("dV", to_np(dv), ref["dv"], dtype)
    else:
        O, L = oracle.attn_fwd(q, k, v, scale, causal, window)
        compare("O", to_np(o), O, dtype)
        compare("L", to_np(lse), L, dtype)

"""Seeded input draws.  Q, K, V, dO are drawn in that order as float32 N(0,1) from a CPU
torch.Generator, then rounded to the workload dtype (round-to-nearest-even for bf16 and
fp16).
The same tensors go to the GPU path and, converted to float64, to the oracle."""
import torch

from .configs import Config

_DT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def make_inputs_like(B, T, H, HKV, D, dtype="f32", seed=0):
    g = torch.Generator("cpu").manual_seed(int(seed))
    q = torch.randn(B, T, H, D, generator=g, dtype=torch.float32)
    k = torch.randn(B, T, HKV, D, generator=g, dtype=torch.float32)
    v = torch.randn(B, T, HKV, D, generator=g, dtype=torch.float32)
    do = torch.randn(B, T, H, D, generator=g, dtype=torch.float32)
    dt = _DT[dtype]
    return q.to(dt), k.to(dt), v.to(dt), do.to(dt)


def make_inputs(cfg: Config, seed=None):
    """(q, k, v, do) CPU tensors in [B,T,H,D] / [B,T,HKV,D] layout for a workload."""
    return make_inputs_like(cfg.B, cfg.T, cfg.H, cfg.HKV, cfg.D, cfg.dtype,
                            cfg.seed if seed is None else seed)

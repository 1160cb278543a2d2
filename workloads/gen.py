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


def make_qk_packed(tokens, heads, D, dtype="bf16", seed=0):
    """A packed QK projection [tokens, 2 * heads, D] (query heads first): seeded N(0, 1)
    draws rounded to the dtype."""
    g = torch.Generator("cpu").manual_seed(int(seed))
    return torch.randn(tokens, 2 * heads, D, generator=g, dtype=torch.float32).to(_DT[dtype])


def rotary_tables(tokens, D, rotary_dim, base=10000.0, pos0=0, halves=1, dtype=torch.float32):
    """Rotary factor tables [tokens, halves * D] (float32 by default): pair i < rotary_dim / 2 of
    token t turns by (pos0 + t) * base^(-2i / rotary_dim), so factor1 = cos on both elements of
    the pair and factor2 = -sin on the even one, +sin on the odd one; elements from rotary_dim
    on are stationary (factor1 = 1, factor2 = 0).  halves = 2 repeats the row (double-width
    tables of paired heads)."""
    npair = rotary_dim // 2
    freq = base ** (-2.0 * torch.arange(npair, dtype=torch.float64) / rotary_dim)
    ang = (pos0 + torch.arange(tokens, dtype=torch.float64))[:, None] * freq[None, :]
    f1 = torch.ones(tokens, D, dtype=torch.float64)
    f2 = torch.zeros(tokens, D, dtype=torch.float64)
    f1[:, 0:rotary_dim:2] = torch.cos(ang)
    f1[:, 1:rotary_dim:2] = torch.cos(ang)
    f2[:, 0:rotary_dim:2] = -torch.sin(ang)
    f2[:, 1:rotary_dim:2] = torch.sin(ang)
    f1, f2 = f1.repeat(1, halves), f2.repeat(1, halves)
    return f1.to(dtype), f2.to(dtype)

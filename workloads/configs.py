"""The five attention workloads (shapes, dtypes, tiles, seeds) and their FLOP accounting.

Shapes follow the pages' workloads: FlashMetal's fixed kernel shape (query/key tiles of 32,
embedding 8, sequence 1024, 8 heads) seeds the fp32 cases, forge's flash_attention.metal header
sizes the memory argument at batch 64 x T 1024 x 8 heads, and the bf16 cases are the causal
(GQA, windowed) shapes the throughput metric is quoted on.  Every tensor is i.i.d. N(0,1).
"""
from dataclasses import dataclass, field
import math


@dataclass(frozen=True)
class Config:
    name: str
    dtype: str          # "f32" or "bf16": dtype of Q, K, V, O, dO
    B: int
    H: int
    HKV: int
    T: int
    D: int
    causal: bool = True
    window: int = 0     # keys kept including self; 0 = no window
    tiles: tuple = (0, 0)   # (Bq, Bk); (0, 0) = library default
    seed: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    def describe(self) -> str:
        w = f", window={self.window}" if self.window else ""
        t = f", tiles {self.tiles[0]}x{self.tiles[1]}" if self.tiles != (0, 0) else ""
        return (f"{'causal ' if self.causal else ''}{self.dtype} B={self.B} H={self.H} "
                f"HKV={self.HKV} T={self.T} D={self.D}{w}{t}")


CONFIGS = {
    "C1": Config("C1", "f32", 1, 2, 2, 128, 64, True, 0, (32, 32), 1),
    "C2a": Config("C2a", "f32", 64, 8, 8, 1024, 8, True, 0, (64, 16), 2),
    "C2b": Config("C2b", "f32", 64, 8, 8, 1024, 64, True, 0, (64, 16), 3),
    "C3": Config("C3", "bf16", 8, 16, 16, 2048, 64, True, 0, (0, 0), 4),
    "C4": Config("C4", "bf16", 4, 32, 8, 4096, 128, True, 0, (0, 0), 5),
    "C5": Config("C5", "bf16", 1, 32, 8, 16384, 128, True, 1024, (0, 0), 6),
}


def get_config(name: str) -> Config:
    return CONFIGS[name]


def fwd_flops(cfg: Config) -> float:
    """Metric convention: 4*B*H*T^2*D for the forward, halved when causal."""
    f = 4.0 * cfg.B * cfg.H * cfg.T * cfg.T * cfg.D
    return f / 2 if cfg.causal else f


def bwd_flops(cfg: Config) -> float:
    """Metric convention: the backward counts 2.5x the forward."""
    return 2.5 * fwd_flops(cfg)


def visible_pairs(T: int, causal: bool, window: int) -> int:
    """Number of (query, key) pairs a row-wise mask keeps, per (batch, head)."""
    total = 0
    for i in range(T):
        hi = i if causal else T - 1
        lo = max(0, i - window + 1) if window > 0 else 0
        total += max(0, hi - lo + 1)
    return total


def window_aware_fwd_flops(cfg: Config) -> float:
    """4*D FLOP per visible score (2*D for Q.K, 2*D for P.V)."""
    return 4.0 * cfg.B * cfg.H * cfg.D * visible_pairs(cfg.T, cfg.causal, cfg.window)

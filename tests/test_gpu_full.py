"""Full-size workloads in the launch configuration bench.py times (GPU).

The oracle cannot afford every (batch, KV-head) group at these sizes, so each test compares
every output element of a few seeded, sampled groups (all their query heads) with the fp64
oracle, and checks invariants that hold exactly for every group: softmax shift invariance
gives sum_j dK_j = 0, rows of P summing to one give sum_j dV_j = sum over the group's heads
and rows of dO.  Outputs are pre-filled with NaN so an unwritten element fails."""
import math

import numpy as np
import pytest
import torch

import oracle
from parity import compare, gpu_bwd, gpu_fwd, log, to_np
from workloads import CONFIGS, make_inputs

pytestmark = pytest.mark.gpu

# groups sampled per config: first, last and one seeded interior group
N_GROUPS = {"C2a": 3, "C2b": 3, "C3": 3, "C4": 2, "C5": 1}


def sampled_groups(cfg, n):
    rng = np.random.default_rng(cfg.seed)
    all_g = [(b, g) for b in range(cfg.B) for g in range(cfg.HKV)]
    pick = [all_g[0], all_g[-1]] + [all_g[int(i)] for i in rng.integers(0, len(all_g), 4)]
    out = []
    for p in pick:
        if p not in out:
            out.append(p)
    return out[:n]


@pytest.mark.parametrize("name", ["C2a", "C2b", "C3", "C4", "C5"])
def test_full_size(name):
    cfg = CONFIGS[name]
    log(f"full-size {name}: {cfg.describe()}")
    q, k, v, do = make_inputs(cfg)
    o, lse, dev = gpu_fwd(q, k, v, cfg.causal, cfg.window, cfg.scale, cfg.tiles)
    dq, dk, dv = gpu_bwd(dev, o, lse, do, cfg.causal, cfg.window, cfg.scale, cfg.tiles)
    O, L, dQ, dK, dV = (to_np(t) for t in (o, lse, dq, dk, dv))
    del o, lse, dq, dk, dv, dev
    torch.cuda.empty_cache()
    for t in (O, L, dQ, dK, dV):
        assert np.isfinite(t).all()

    # invariants over every group
    dO = do.float().numpy().astype(np.float64)
    rep = cfg.H // cfg.HKV
    sdk = dK.sum(axis=1)                       # [B, HKV, D]
    assert np.abs(sdk).max() <= 1e-2 * np.abs(dK).sum(axis=1).max() + 1e-6
    sdo = dO.reshape(cfg.B, cfg.T, cfg.HKV, rep, cfg.D).sum(axis=(1, 3))
    assert np.abs(dV.sum(axis=1) - sdo).max() <= 1e-2 * np.abs(sdo).max() + 1e-3

    # every element of the sampled groups
    groups = sampled_groups(cfg, N_GROUPS[name])
    log(f"  oracle on groups {groups}")
    ref = oracle.attn_bwd(q, k, v, do, cfg.scale, cfg.causal, cfg.window, groups=groups)
    for b, g in groups:
        hs = slice(g * rep, (g + 1) * rep)
        compare(f"O{(b, g)}", O[b, :, hs], ref["o"][b, :, hs], cfg.dtype)
        compare(f"L{(b, g)}", L[b, hs], ref["lse"][b, hs], cfg.dtype)
        compare(f"dQ{(b, g)}", dQ[b, :, hs], ref["dq"][b, :, hs], cfg.dtype)
        compare(f"dK{(b, g)}", dK[b, :, g], ref["dk"][b, :, g], cfg.dtype)
        compare(f"dV{(b, g)}", dV[b, :, g], ref["dv"][b, :, g], cfg.dtype)


def test_bitwise_deterministic():
    """Two runs of fwd + bwd give identical bits (no atomics, fixed reduction order)."""
    cfg = CONFIGS["C3"]
    q, k, v, do = make_inputs(cfg)
    runs = []
    for _ in range(2):
        o, lse, dev = gpu_fwd(q, k, v, cfg.causal, cfg.window, cfg.scale)
        dq, dk, dv = gpu_bwd(dev, o, lse, do, cfg.causal, cfg.window, cfg.scale)
        runs.append([t.cpu() for t in (o, lse, dq, dk, dv)])
    for a, b in zip(*runs):
        assert torch.equal(a, b)

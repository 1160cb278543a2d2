"""Seeded inputs and FLOP / byte accounting (CPU only)."""
import torch

from workloads import CONFIGS, make_inputs, make_inputs_like, fwd_flops, bwd_flops, visible_pairs
from workloads.configs import window_aware_fwd_flops


def test_inputs_are_seeded_and_shaped():
    a = make_inputs_like(2, 5, 4, 2, 8, "bf16", 3)
    b = make_inputs_like(2, 5, 4, 2, 8, "bf16", 3)
    c = make_inputs_like(2, 5, 4, 2, 8, "bf16", 4)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    assert not torch.equal(a[0], c[0])
    q, k, v, do = a
    assert q.shape == (2, 5, 4, 8) and k.shape == (2, 5, 2, 8) and v.shape == k.shape
    assert do.shape == q.shape and q.dtype == torch.bfloat16


def test_bf16_inputs_are_rne_of_f32_draws():
    q32 = make_inputs_like(1, 7, 2, 1, 16, "f32", 9)[0]
    q16 = make_inputs_like(1, 7, 2, 1, 16, "bf16", 9)[0]
    assert torch.equal(q32.to(torch.bfloat16), q16)


def test_metric_flops():
    c4 = CONFIGS["C4"]
    assert fwd_flops(c4) == 4 * 4 * 32 * 4096 ** 2 * 128 / 2 == 549755813888.0
    assert bwd_flops(c4) == 2.5 * fwd_flops(c4)
    assert fwd_flops(CONFIGS["C1"]) == 4 * 1 * 2 * 128 ** 2 * 64 / 2


def test_window_visible_pairs():
    assert visible_pairs(16384, True, 1024) == 16253440
    assert visible_pairs(8, True, 0) == 36
    assert visible_pairs(8, False, 0) == 64
    c5 = CONFIGS["C5"]
    assert abs(window_aware_fwd_flops(c5) / fwd_flops(c5) - 0.1211) < 1e-3


def test_unfused_probability_bytes():
    """forge flash_attention.metal header: materialised probabilities cost B*H*T^2 floats, about
    2.1 GB at batch 64, T 1024, 8 heads; the fused path keeps B*H*T floats of L."""
    assert 64 * 8 * 1024 ** 2 * 4 == 2_147_483_648
    assert 64 * 8 * 1024 * 4 == 2 * 1024 ** 2

"""HIP path vs the fp64 oracle, element by element, on seeded inputs small enough for the
oracle to finish in seconds but spanning several tiles and a ragged tail (GPU)."""
import pytest
import torch

from parity import check_case

pytestmark = pytest.mark.gpu

MASKS = [(True, 0), (True, 7), (True, 100), (False, 0), (False, 13), (True, 1)]


def test_c1_exact_config():
    """Causal MHA fp32, B=1, H=HKV=2, T=128, D=64, 32x32 tiles."""
    check_case(1, 128, 2, 2, 64, "f32", True, 0, seed=1, tiles=(32, 32))


@pytest.mark.parametrize("tiles", [(32, 32), (64, 16), (64, 64), (32, 64), (64, 32), (32, 16)])
@pytest.mark.parametrize("causal,window", MASKS)
def test_f32_tiles_and_masks(tiles, causal, window):
    check_case(1, 100, 4, 2, 64, "f32", causal, window, seed=31, tiles=tiles)


@pytest.mark.parametrize("D", list(range(8, 129, 8)))
def test_f32_every_head_dim(D):
    check_case(1, 129, 2, 1, D, "f32", True, 0, seed=40 + D, tiles=(64, 16))


@pytest.mark.parametrize("tiles", [(32, 32), (64, 16), (64, 64), (32, 16)])
@pytest.mark.parametrize("causal,window", MASKS)
def test_f32_d8_tiles_and_masks(tiles, causal, window):
    """D = 8: the forward's V tile carries ones in its padding column, so the row sums come
    out of the PV products (rescaled with O)."""
    check_case(1, 100, 4, 2, 8, "f32", causal, window, seed=36, tiles=tiles)


@pytest.mark.parametrize("T", [1, 2, 17, 130])
def test_f32_d8_ragged_lengths(T):
    check_case(2, T, 4, 1, 8, "f32", True, 3 if T > 17 else 0, seed=37 + T, tiles=(64, 16))


@pytest.mark.parametrize("T", [1, 2, 17, 257])
def test_f32_ragged_lengths(T):
    check_case(2, T, 8, 2, 32, "f32", True, 5 if T > 17 else 0, seed=50 + T)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("T", [1, 100, 257, 640])
@pytest.mark.parametrize("causal,window", MASKS)
def test_bf16_forward(D, T, causal, window):
    check_case(1, T, 8, 2, D, "bf16", causal, window, seed=60 + T + D, backward=False)


@pytest.mark.parametrize("H,HKV", [(4, 4), (8, 1), (8, 4), (16, 2)])
def test_bf16_forward_gqa(H, HKV):
    check_case(2, 300, H, HKV, 128, "bf16", True, 0, seed=70 + H * HKV, backward=False)


def test_bf16_forward_large_scale_value():
    """A scale above 1 (so scale * log2(e) > 1) with masked rows in the first key block."""
    check_case(1, 200, 4, 2, 64, "bf16", True, 3, seed=80, backward=False, scale=1.7)


def test_f32_large_scale_value():
    check_case(1, 70, 2, 2, 16, "f32", True, 3, seed=81, scale=2.5)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("T", [1, 100, 257])
@pytest.mark.parametrize("causal,window", [(True, 0), (True, 7), (False, 0), (False, 13)])
def test_bf16_backward(D, T, causal, window):
    check_case(1, T, 8, 2, D, "bf16", causal, window, seed=100 + T + D)


@pytest.mark.parametrize("H,HKV", [(4, 4), (8, 1), (16, 2)])
def test_bf16_backward_gqa(H, HKV):
    check_case(2, 384, H, HKV, 128, "bf16", True, 0, seed=110 + H * HKV)


def test_bf16_backward_long_window():
    check_case(1, 1100, 4, 1, 128, "bf16", True, 300, seed=120)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("T", [1, 100, 257, 640])
@pytest.mark.parametrize("causal,window", [(True, 0), (True, 7), (False, 0), (False, 13)])
def test_f16_forward_backward(D, T, causal, window):
    check_case(1, T, 8, 2, D, "f16", causal, window, seed=130 + T + D)


@pytest.mark.parametrize("H,HKV", [(4, 4), (8, 1), (16, 2)])
def test_f16_gqa(H, HKV):
    check_case(2, 384, H, HKV, 128, "f16", True, 0, seed=140 + H * HKV)


def test_f16_forward_large_scale_value():
    """As the bf16 case: scale above 1, masked rows in the first key block (forward; the
    absolute bounds are set for the 1/sqrt(D) scale the workloads use)."""
    check_case(1, 200, 4, 2, 64, "f16", True, 3, seed=150, backward=False, scale=1.7)


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f16", 64)])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("window", [31, 32, 33, 63, 64, 65, 128, 129])
def test_window_at_block_edges(dtype, D, causal, window):
    """Windows one key shorter or longer than a block (32 keys in the forward and per dK/dV
    query block, 64 in dQ): where each wave's precomputed FULL blocks, which skip the class
    test and the mask, begin and end."""
    check_case(1, 300, 4, 2, D, dtype, causal, window, seed=150 + window)


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("bf16", 64), ("f16", 128)])
@pytest.mark.parametrize("window", [1, 4, 5, 15, 16, 17, 47, 48, 49])
def test_window_at_tile_edges(dtype, D, window):
    """Windows around the 16-key and 4-key granules of the MFMA tiles (a 16x16 accumulator tile
    holds 16 keys, 4 per lane row) and T around the 16-row query tiles: a key index off by one
    inside a tile moves a masked score across the window edge."""
    for T in (47, 49):
        check_case(1, T, 4, 2, D, dtype, True, window, seed=300 + window + T)

"""A seeded sweep of random configurations (GPU): every output of the forward and backward
against the fp64 oracle, element by element, at the dtype's tolerance.  The configurations are
drawn once from a fixed generator, so the sweep is the same on every run; it mixes what the
targeted tests vary one at a time — dtype, head dim, batch, ragged lengths, GQA ratio, causal /
window / neither, and the fp32 path's tilings."""
import numpy as np
import pytest

from parity import check_case

pytestmark = pytest.mark.gpu

F32_TILES = [(32, 32), (64, 16), (64, 64), (32, 64), (64, 32), (32, 16)]


def _cases(n=32, seed=20261203):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dtype = ["bf16", "f16", "f32"][i % 3]
        D = int(rng.choice([64, 128])) if dtype != "f32" else int(8 * rng.integers(1, 17))
        rep = int(rng.choice([1, 2, 4, 8]))
        HKV = int(rng.integers(1, 4))
        B = int(rng.integers(1, 4))
        T = int(rng.integers(1, 700))
        mode = int(rng.integers(0, 4))   # causal, causal + window, window only, neither
        causal = mode in (0, 1)
        window = int(rng.integers(1, T + 8)) if mode in (1, 2) else 0
        tiles = F32_TILES[int(rng.integers(0, len(F32_TILES)))] if dtype == "f32" else (0, 0)
        out.append((B, T, rep * HKV, HKV, D, dtype, causal, window, 1000 + i, tiles))
    return out


@pytest.mark.parametrize("case", _cases(), ids=lambda c: f"{c[5]}-D{c[4]}-T{c[1]}-s{c[8]}")
def test_random_configuration(case):
    B, T, H, HKV, D, dtype, causal, window, seed, tiles = case
    check_case(B, T, H, HKV, D, dtype, causal, window, seed=seed, tiles=tiles)

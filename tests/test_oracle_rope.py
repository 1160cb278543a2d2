"""Pins of the QK RMS-norm + rotary oracle (CPU): an independent library RMS-norm, the
relative-position property of rotary embeddings, norm preservation, the paired-head remap as a
reshape, and the key offset against the previous token's normalised row."""
import numpy as np
import pytest
import torch

import oracle
from workloads import make_qk_packed, rotary_tables

EPS = 2.0 ** -23
F64 = torch.float64   # exact rotations for the closed forms


def lib_rms_norm(x):
    """torch's own rms_norm in fp64 (no weight)."""
    x = torch.as_tensor(x, dtype=torch.float64)
    return torch.nn.functional.rms_norm(x, (x.shape[-1],), eps=EPS).numpy()


def check_identity_tables_give_rms_norm(ora):
    qk = make_qk_packed(5, 3, 16, "f32", seed=1)
    f1, f2 = torch.ones(5, 16), torch.zeros(5, 16)
    q, k = ora.qk_norm_rope(qk, f1, f2, 3, 16)
    want = lib_rms_norm(qk.double())
    assert np.allclose(q, want[:, :3], atol=1e-14, rtol=0)
    assert np.allclose(k, want[:, 3:], atol=1e-14, rtol=0)


def check_relative_position(ora):
    for rotary_dim in (16, 8):
        _relative_position(ora, rotary_dim)


def _relative_position(ora, rotary_dim):
    """Rotated query t1 . rotated key t2 depends on t2 - t1 only: shifting every position by
    s leaves all dot products unchanged (they do change with the distance)."""
    tokens, heads, D = 6, 2, 16
    qk = make_qk_packed(tokens, heads, D, "f32", seed=2)
    # the same vector at every token, so only the rotation differs between tokens
    qk = qk[:1].repeat(tokens, 1, 1)
    dots = []
    for pos0 in (0, 5):
        f1, f2 = rotary_tables(tokens, D, rotary_dim, pos0=pos0, dtype=F64)
        q, k = ora.qk_norm_rope(qk, f1, f2, heads, rotary_dim)
        dots.append(np.einsum("thd,shd->hts", q, k))
    assert np.allclose(dots[0], dots[1], atol=1e-12, rtol=0)
    # equal along diagonals t2 - t1 = const, different across them
    d = dots[0][0]
    assert np.allclose(np.diag(d, 1), np.diag(d, 1)[0], atol=1e-12)
    assert not np.allclose(d[0, 0], d[0, 3], atol=1e-6)


def check_rotation_keeps_the_norm(ora):
    tokens, heads, D = 7, 2, 32
    qk = make_qk_packed(tokens, heads, D, "f32", seed=3)
    f1, f2 = rotary_tables(tokens, D, D, pos0=3, dtype=F64)
    q, k = ora.qk_norm_rope(qk, f1, f2, heads, D)
    x = qk.double().numpy()
    ms = (x * x).mean(-1)
    want = ms / (ms + EPS)
    assert np.allclose((q * q).mean(-1), want[:, :heads], atol=1e-13, rtol=0)
    assert np.allclose((k * k).mean(-1), want[:, heads:], atol=1e-13, rtol=0)


def check_paired_is_a_reshape(ora):
    """With both halves of the double-width tables equal, paired output = the unpaired output
    [tokens, heads, D] viewed as [tokens, 2, heads/2, D] and flattened to [2 tokens, heads/2, D];
    zeroing the second half of the tables zeroes exactly the odd logical heads."""
    tokens, heads, D = 4, 4, 8
    qk = make_qk_packed(tokens, heads, D, "f32", seed=4)
    f1, f2 = rotary_tables(tokens, D, D, pos0=1)
    q1, k1 = ora.qk_norm_rope(qk, f1, f2, heads, D)
    f1p, f2p = rotary_tables(tokens, D, D, pos0=1, halves=2)
    q2, k2 = ora.qk_norm_rope(qk, f1p, f2p, heads, D, paired=True)
    assert np.array_equal(q2, q1.reshape(tokens, 2, heads // 2, D).reshape(2 * tokens, heads // 2, D))
    assert np.array_equal(k2, k1.reshape(tokens, 2, heads // 2, D).reshape(2 * tokens, heads // 2, D))
    f1z, f2z = f1p.clone(), f2p.clone()
    f1z[:, D:] = 0
    f2z[:, D:] = 0
    q3, _ = ora.qk_norm_rope(qk, f1z, f2z, heads, D, paired=True)
    q3 = q3.reshape(tokens, 2, heads // 2, D).reshape(tokens, heads, D)
    assert (q3[:, 1::2] == 0).all()
    assert np.array_equal(q3[:, 0::2], q1[:, 0::2])


def check_key_offset_takes_previous_token(ora):
    tokens, heads, D, rd = 5, 2, 16, 10
    qk = make_qk_packed(tokens, heads, D, "f32", seed=5)
    f1, f2 = rotary_tables(tokens, D, rd)
    q0, k0 = ora.qk_norm_rope(qk, f1, f2, heads, rd)
    q1, k1 = ora.qk_norm_rope(qk, f1, f2, heads, rd, key_offset=True)
    norm = lib_rms_norm(qk.double())
    assert np.array_equal(q1, q0)                               # queries untouched
    assert np.array_equal(k1[0], k0[0])                         # first token keeps its own
    assert np.array_equal(k1[:, :, :rd], k0[:, :, :rd])         # rotating part untouched
    assert np.allclose(k1[1:, :, rd:], norm[:-1, heads:, rd:], atol=1e-14, rtol=0)


CHECKS = [check_identity_tables_give_rms_norm, check_relative_position,
          check_rotation_keeps_the_norm, check_paired_is_a_reshape,
          check_key_offset_takes_previous_token]


@pytest.mark.parametrize("check", CHECKS, ids=lambda c: c.__name__)
def test_rope_oracle_pin(check):
    check(oracle)


ROPE_MUTANTS = {
    "no_pair_swap": ("xs = swap_pairs(xn)", "xs = xn"),
    "roll_instead_of_swap": ("xs = swap_pairs(xn)", "xs = np.roll(xn, 1, axis=-1)"),
    "paired_half_by_output_token": ("(lh % 2) * D", "(lh // (heads // 2)) * D"),
    "key_offset_same_token": ("y[rotary_dim:] = xn[t - 1, ih, rotary_dim:]",
                              "y[rotary_dim:] = xn[t, ih, rotary_dim:]"),
    "norm_without_mean": ("np.mean(x * x, axis=-1, keepdims=True)",
                          "np.sum(x * x, axis=-1, keepdims=True)"),
}


@pytest.mark.parametrize("name", sorted(ROPE_MUTANTS))
def test_rope_mutant_is_caught(name):
    """A plausible mistake planted in the oracle's source fails at least one pin."""
    import os
    import types
    old, new = ROPE_MUTANTS[name]
    src = open(os.path.join(os.path.dirname(oracle.__file__), "rope.py")).read()
    assert old in src
    src = src.replace(old, new).replace("from .attention import _f64",
                                        "from oracle.attention import _f64")
    mod = types.ModuleType("rope_mutant")
    exec(compile(src, "rope_mutant", "exec"), mod.__dict__)
    failures = 0
    for check in CHECKS:
        try:
            check(mod)
        except (AssertionError, ValueError):
            failures += 1
    assert failures > 0, name

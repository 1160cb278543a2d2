"""fp64 reference for the QK RMS-norm + rotary prologue that feeds attention its Q and K.
TEST INFRASTRUCTURE ONLY (see the package docstring).

Source (web page, cited by title and section): modded-nanogpt "qkv_rope.py", the module
docstring and qk_norm_rope_forward with its forward kernel.  What it computes, in its order:
  * the input is one packed QK projection [tokens, 2 * heads, qk_dim]: input heads below
    `heads` are query heads, the rest key heads;
  * each row x (one token, one input head) is RMS-normalised in fp32 with no weight:
    x * rsqrt(mean(x^2) + eps), eps = 2^-23 (the fp32 eps of torch's rms_norm);
  * the rotary step mixes each element with its pair partner (elements 2i and 2i + 1 swap):
    y = factor1 * x_norm + factor2 * x_norm_swapped, with per-token factor tables given as
    inputs (a rotation has factor1 = cos, factor2 = -sin on even and +sin on odd elements);
  * paired heads: logical head h of token t goes to output token 2t + h // (heads / 2), output
    head h % (heads / 2), and reads the second half of a double-width factor row when h is
    odd;
  * key offset: for a key head of a token t > 0 the stationary elements (index >= rotary_dim)
    are the previous token's normalised row instead;
  * queries and keys are stored to two separate outputs.
Plain loops over rows; float64 throughout.
"""
import numpy as np

from .attention import _f64

EPS = 2.0 ** -23


def rms_normalise(x, eps=EPS):
    """x / sqrt(mean(x^2) + eps) along the last axis."""
    x = _f64(x)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def swap_pairs(x):
    """Elements 2i and 2i + 1 exchanged along the last axis."""
    y = np.empty_like(x)
    y[..., 0::2] = x[..., 1::2]
    y[..., 1::2] = x[..., 0::2]
    return y


def qk_norm_rope(qk, factor1, factor2, heads, rotary_dim, paired=False, key_offset=False,
                 eps=EPS):
    """(out_q, out_k) in fp64 from qk [tokens, 2*heads, D] and factor tables
    [tokens, D * (2 if paired else 1)]; each output is [tokens, heads, D], or
    [2*tokens, heads/2, D] when paired."""
    qk = _f64(qk)
    f1, f2 = _f64(factor1), _f64(factor2)
    tokens, heads2, D = qk.shape
    if heads2 != 2 * heads or (paired and key_offset) or (paired and heads % 2):
        raise ValueError("bad qk_norm_rope arguments")
    if f1.shape != (tokens, D * (2 if paired else 1)) or f2.shape != f1.shape:
        raise ValueError("bad factor table shape")
    xn = rms_normalise(qk, eps)
    xs = swap_pairs(xn)
    shape = (2 * tokens, heads // 2, D) if paired else (tokens, heads, D)
    out_q = np.zeros(shape)
    out_k = np.zeros(shape)
    for t in range(tokens):
        for ih in range(heads2):
            lh = ih % heads
            if paired:
                ot, oh, off = 2 * t + lh // (heads // 2), lh % (heads // 2), (lh % 2) * D
            else:
                ot, oh, off = t, lh, 0
            y = f1[t, off:off + D] * xn[t, ih] + f2[t, off:off + D] * xs[t, ih]
            if key_offset and ih >= heads and t > 0:
                y[rotary_dim:] = xn[t - 1, ih, rotary_dim:]
            (out_q if ih < heads else out_k)[ot, oh] = y
    return out_q, out_k

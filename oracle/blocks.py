"""Brute-force block classification for tiled causal / sliding-window attention.
TEST INFRASTRUCTURE ONLY (see the package docstring).

A tiling cuts the T x T keep-matrix into Bq x Bk blocks (query tile i, key block j).  Each
block is SKIP (nothing visible: its scores are never computed), FULL (every in-range element
visible: no mask test needed) or PARTIAL (a per-element test is needed).  The classification
here is read straight off the materialised mask; nothing is derived from block arithmetic.

For a PARTIAL block the mask is rebuilt from the single integer off = i*Bq - j*Bk:
keep (r, c) iff c <= r + off (causal), c >= r + off - W + 1 (window) and the global indices are
< T.  The Graphcore page (flash_attention_qkv_packed.cpp, getTriuOffsetSequence and its
docstring; makeDynamicCausalMaskBlocks) keeps one pre-built mask per distinct value of off+1
and walks them cyclically; triu_offset_sequence() reproduces that cycle by walking the block
diagonal, so a test can compare it with the brute-force list.
"""
import numpy as np

from .attention import visible_mask

SKIP, FULL, PARTIAL = 0, 1, 2


def _cdiv(a, b):
    return -(-a // b)


def classify_blocks(T, Bq, Bk, causal, window, Tk=None):
    """[ceil(T/Bq), ceil(Tk/Bk)] int array of SKIP/FULL/PARTIAL from the materialised mask of
    T query rows against Tk keys (Tk = T by default).

    A block that sticks out past Tk counts as PARTIAL when any of its in-range elements are
    visible, because the out-of-range keys must still be excluded."""
    Tk = T if Tk is None else Tk
    vis = visible_mask(T, causal, window, Tk=Tk)
    nq, nk = _cdiv(T, Bq), _cdiv(Tk, Bk)
    out = np.zeros((nq, nk), dtype=np.int64)
    for i in range(nq):
        for j in range(nk):
            blk = vis[i * Bq:(i + 1) * Bq, j * Bk:(j + 1) * Bk]
            if not blk.any():
                out[i, j] = SKIP
            elif blk.all() and (j + 1) * Bk <= Tk:
                out[i, j] = FULL
            else:
                out[i, j] = PARTIAL
    return out


def block_keep_mask(i, j, Bq, Bk, T, causal, window):
    """Bq x Bk keep mask of block (i, j) rebuilt from off = i*Bq - j*Bk alone (plus T)."""
    off = i * Bq - j * Bk
    r = np.arange(Bq)[:, None]
    c = np.arange(Bk)[None, :]
    keep = np.ones((Bq, Bk), dtype=bool)
    if causal:
        keep &= c <= r + off
    if window > 0:
        keep &= c >= r + off - window + 1
    keep &= (i * Bq + r < T) & (j * Bk + c < T)
    return keep


def kv_block_range(i, Bq, Bk, T, causal, window, Tk=None):
    """(first, last+1) key blocks of query tile i that hold any visible element, read off the
    materialised mask; (0, 0) when the tile sees nothing."""
    cls = classify_blocks(T, Bq, Bk, causal, window, Tk)[i]
    live = np.nonzero(cls != SKIP)[0]
    if live.size == 0:
        return 0, 0
    return int(live[0]), int(live[-1]) + 1


def partial_offsets_in_loop_order(T, Bq, Bk):
    """off+1 of every causal PARTIAL block, query tiles outer and key blocks inner."""
    cls = classify_blocks(T, Bq, Bk, True, 0)
    seq = []
    for i in range(cls.shape[0]):
        for j in range(cls.shape[1]):
            if cls[i, j] == PARTIAL:
                seq.append(i * Bq - j * Bk + 1)
    return seq


def triu_offset_sequence(Bq, Bk, max_steps=1_000_000):
    """One period of the mask offsets (off+1) that causal PARTIAL blocks show, in the order a
    query-outer / key-inner loop meets them.

    Walk the block diagonal from block (0, 0) (offset 1).  From block (i, j) go down to
    (i+1, j) unless that block lies entirely below the diagonal (it would need no mask), in
    which case go right to (i, j+1).  Every block reached that is not entirely above the
    diagonal is a masked block; the walk has closed its period when the offset is 1 again.
    With a key block of a single column the walk never returns to offset 1 (see the tests);
    it then stops after max_steps and raises.
    """
    i, j = 0, 0
    seq = [1]
    for _ in range(max_steps):
        below = (i + 1) * Bq - j * Bk + 1 > Bk - 1   # (i+1, j) needs no mask
        if below:
            j += 1
        else:
            i += 1
        k = i * Bq - j * Bk + 1
        if k == 1:
            return seq
        if k >= 2 - Bq:                                # block is executed at all
            seq.append(k)
    raise RuntimeError(f"offset walk did not close for Bq={Bq}, Bk={Bk}")

"""Block classification of the oracle against brute-force masks, the Graphcore page's worked
mask pictures and its cyclic mask-offset scheme (CPU only)."""
import math
import os

import numpy as np
import pytest

import oracle
from oracle import SKIP, FULL, PARTIAL

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "graphcore_triu_blocks.txt")


def load_pictures():
    cases, cur = [], None
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("case"):
                n, bq, bk = map(int, line.split()[1:])
                cur = (n, bq, bk, [])
                cases.append(cur)
            else:
                cur[3].append([int(x) for x in line.split()])
    return [(n, bq, bk, np.array(rows, dtype=bool)) for n, bq, bk, rows in cases]


def test_pictures_parse():
    pics = load_pictures()
    assert [(n, bq, bk) for n, bq, bk, _ in pics] == [(4, 2, 2), (6, 2, 3), (8, 2, 4)]
    for n, _, _, m in pics:
        assert m.shape == (n, n)


@pytest.mark.parametrize("case", range(3))
def test_block_masks_match_pictures(case):
    """Cut each pictured matrix into its Bq x Bk blocks.  The elements strictly above the
    diagonal are the ones causal attention drops, so every block's drop pattern must equal the
    complement of the oracle's keep mask rebuilt from off = i*Bq - j*Bk alone."""
    n, bq, bk, pic = load_pictures()[case]
    diag = np.eye(n, dtype=bool)
    dropped = pic & ~diag
    for i in range(n // bq):
        for j in range(n // bk):
            blk = dropped[i * bq:(i + 1) * bq, j * bk:(j + 1) * bk]
            keep = oracle.block_keep_mask(i, j, bq, bk, n, True, 0)
            assert np.array_equal(~blk, keep), (i, j)


def _picture_partial_offsets(n, bq, bk, pic):
    """off+1 of each block of the picture that holds both kept and dropped elements, read off
    the picture: in a masked block the row rr keeps its first (rr + off + 1) columns."""
    dropped = pic & ~np.eye(n, dtype=bool)
    out = []
    for i in range(n // bq):
        for j in range(n // bk):
            blk = dropped[i * bq:(i + 1) * bq, j * bk:(j + 1) * bk]
            if blk.any() and not blk.all():
                kept_per_row = (~blk).sum(axis=1)
                rr = int(np.nonzero((kept_per_row > 0) & (kept_per_row < bk))[0][0])
                out.append(int(kept_per_row[rr]) - rr)
    return out


def test_picture_offset_claims():
    """The docstring's claims about its three pictures: square blocks need one mask pattern;
    2x3 blocks meet the diagonal with a different pattern each time; with 2x4 blocks the two
    upper-left masked blocks repeat as the two lower-right ones."""
    pics = load_pictures()
    offs = {(bq, bk): _picture_partial_offsets(n, bq, bk, p) for n, bq, bk, p in pics}
    assert len(set(offs[(2, 2)])) == 1
    assert len(set(offs[(2, 3)])) == len(offs[(2, 3)]) >= 3
    assert len(offs[(2, 4)]) == 4 and offs[(2, 4)][:2] == offs[(2, 4)][2:]
    for n, bq, bk, p in pics:
        assert oracle.partial_offsets_in_loop_order(n, bq, bk) == offs[(bq, bk)]
        cyc = oracle.triu_offset_sequence(bq, bk)
        o = offs[(bq, bk)]
        assert o == [cyc[m % len(cyc)] for m in range(len(o))]


@pytest.mark.parametrize("bq,bk", [(bq, bk) for bq in (1, 2, 3, 4, 5, 8, 16, 32, 64, 128)
                                   for bk in (2, 3, 4, 7, 16, 32, 64, 128)])
def test_offset_walk_matches_brute_force(bq, bk):
    """The diagonal walk's cycle, repeated, is exactly the list of masked-block offsets a
    query-outer / key-inner loop meets, for T a multiple of both tile sizes (the page asserts
    divisibility)."""
    cyc = oracle.triu_offset_sequence(bq, bk)
    L = math.lcm(bq, bk)
    for m in (1, 2, 3):
        T = m * L
        if T > 1024:
            break
        got = oracle.partial_offsets_in_loop_order(T, bq, bk)
        assert got == [cyc[n % len(cyc)] for n in range(len(got))]


def test_offset_walk_known_cycles():
    assert oracle.triu_offset_sequence(64, 16) == [1, -15, -31, -47]
    assert oracle.triu_offset_sequence(16, 64) == [1, 17, 33, 49]
    assert oracle.triu_offset_sequence(128, 64) == [1, -63]
    assert oracle.triu_offset_sequence(32, 32) == [1]


def test_offset_walk_single_column_keys_never_closes():
    """With Bk = 1 no masked block ever needs an offset of 1 again: the walk does not close."""
    with pytest.raises(RuntimeError):
        oracle.triu_offset_sequence(4, 1, max_steps=10_000)


SWEEP = [(T, bq, bk, c, w) for T in (1, 5, 64, 100, 129, 257)
         for bq, bk in ((32, 32), (64, 16), (16, 64), (128, 64), (64, 64), (7, 3))
         for c, w in ((True, 0), (True, 1), (True, 7), (True, 40), (False, 0), (False, 9))]


@pytest.mark.parametrize("T,bq,bk,causal,window", SWEEP)
def test_rebuilt_masks_match_materialised(T, bq, bk, causal, window):
    """For every block, the mask rebuilt from off (and T) equals the slice of the materialised
    keep matrix bit for bit; SKIP blocks are all-False and FULL blocks all-True."""
    vis = oracle.visible_mask(T, causal, window)
    cls = oracle.classify_blocks(T, bq, bk, causal, window)
    for i in range(cls.shape[0]):
        for j in range(cls.shape[1]):
            keep = oracle.block_keep_mask(i, j, bq, bk, T, causal, window)
            sl = np.zeros((bq, bk), dtype=bool)
            blk = vis[i * bq:(i + 1) * bq, j * bk:(j + 1) * bk]
            sl[:blk.shape[0], :blk.shape[1]] = blk
            assert np.array_equal(keep, sl)
            if cls[i, j] == SKIP:
                assert not keep.any()
            elif cls[i, j] == FULL:
                rows_in = min(bq, T - i * bq)
                assert keep[:rows_in].all()


@pytest.mark.parametrize("T,bq,bk,causal,window", SWEEP[::3])
def test_live_blocks_are_contiguous(T, bq, bk, causal, window):
    """Between a query tile's first and last live key block no block is SKIP, so a kernel may
    loop over one contiguous key-block range."""
    cls = oracle.classify_blocks(T, bq, bk, causal, window)
    for i in range(cls.shape[0]):
        lo, hi = oracle.kv_block_range(i, bq, bk, T, causal, window)
        assert (cls[i, lo:hi] != SKIP).all()
        assert (cls[i, :lo] == SKIP).all() and (cls[i, hi:] == SKIP).all()

"""The C-ABI library on the CPU: it loads, exports every declared symbol, rejects invalid
arguments before touching the GPU, and its host-side block classifier (the same header the
kernels use) agrees bit for bit with the oracle's brute-force classification."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import online_softmax_fwd_flash_amd as fa
from online_softmax_fwd_flash_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flash_attn.h")


def declared_symbols():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(flash_attn_\w+)\s*\(", src)))


def test_header_and_exports_agree():
    decl = declared_symbols()
    assert len(decl) >= 12
    assert sorted(_lib.EXPORTS) == decl
    lib = ctypes.CDLL(_lib.LIB_PATH)
    for name in decl:
        assert hasattr(lib, name), name


def test_version_and_strings():
    assert fa.flash_attn_version() == 102
    assert _lib.status_string(0) == "FA_OK"
    assert _lib.status_string(2) == "FA_ERR_UNSUPPORTED"


A = ctypes.c_void_p(0x1000)       # aligned, never dereferenced: every call below fails validation
MIS = ctypes.c_void_p(0x1004)
NUL = ctypes.c_void_p(0)
S0 = ctypes.c_void_p(0)

GOOD = dict(B=1, T=16, H=4, HKV=2, D=64, scale=0.125, causal=1, window=0, dtype=1)


def fwd(ptrs=(A, A, A, A, A), **kw):
    p = dict(GOOD, **kw)
    return _lib.lib().flash_attn_fwd(*ptrs, p["B"], p["T"], p["H"], p["HKV"], p["D"], p["scale"],
                                     p["causal"], p["window"], p["dtype"], S0)


def bwd(ptrs=(A,) * 9, **kw):
    p = dict(GOOD, **kw)
    return _lib.lib().flash_attn_bwd(*ptrs, p["B"], p["T"], p["H"], p["HKV"], p["D"], p["scale"],
                                     p["causal"], p["window"], p["dtype"], S0)


def dq_dvec(ptrs=(A,) * 8, bq=0, bk=0, **kw):
    p = dict(GOOD, **kw)
    return _lib.lib().flash_attn_bwd_dq_dvec(*ptrs, p["B"], p["T"], p["H"], p["HKV"], p["D"],
                                             p["scale"], p["causal"], p["window"], p["dtype"], S0,
                                             bq, bk)


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), 1), (dict(T=0), 1), (dict(H=0), 1), (dict(HKV=0), 1), (dict(D=0), 1),
    (dict(H=6, HKV=4), 1), (dict(window=-1), 1), (dict(scale=float("nan")), 1),
    (dict(scale=float("inf")), 1), (dict(scale=0.0), 1), (dict(scale=-0.5), 1),
    (dict(causal=2), 1), (dict(dtype=7), 1),
    (dict(D=96), 2), (dict(D=32), 2), (dict(dtype=0, D=12), 2), (dict(dtype=0, D=136), 2),
    (dict(T=1 << 30, H=64, D=128), 1),
    (dict(T=1 << 24, H=64, HKV=8, D=128), 1),     # bf16 batch slice of Q reaches 2 GiB
])
def test_fwd_and_bwd_reject_before_launch(kw, code):
    assert fwd(**kw) == code
    assert bwd(**kw) == code
    assert dq_dvec(**kw) == code


@pytest.mark.parametrize("which", range(5))
def test_null_and_misaligned_pointers(which):
    for bad in (NUL, MIS):
        ptrs = [A] * 5
        ptrs[which] = bad
        assert fwd(tuple(ptrs)) == 1
        ptrs9 = [A] * 9
        ptrs9[which + 4] = bad
        assert bwd(tuple(ptrs9)) == 1
        ptrs8 = [A] * 8
        ptrs8[which + 3] = bad
        assert dq_dvec(tuple(ptrs8)) == 1


def test_bad_tiles_rejected():
    L = _lib.lib()
    args = (A, A, A, A, A, 1, 64, 2, 2, 64, 0.125, 1, 0, 0, S0)
    assert L.flash_attn_fwd_ex(*args, 48, 16) == 1
    assert L.flash_attn_fwd_ex(*args, 64, 8) == 1
    args16 = (A, A, A, A, A, 1, 64, 2, 2, 64, 0.125, 1, 0, 1, S0)
    assert L.flash_attn_fwd_ex(*args16, 64, 64) == 1
    assert dq_dvec(bq=64, bk=64) == 1
    assert dq_dvec(bq=128, bk=32) == 1
    assert dq_dvec(dtype=0, bq=48, bk=16) == 1


def test_grad16_rejects_before_launch():
    L = _lib.lib()
    q = _lib.Layout(64 * 4 * 128, 4 * 128, 128)
    k = _lib.Layout(64 * 2 * 128, 2 * 128, 128)
    dims = [1, 64, 64, 4, 2, 128, 0.125, 1, 0, 1, S0]
    dims32 = list(dims); dims32[9] = 0
    assert L.flash_attn_bwd_grad16(*([A] * 9), *dims32, q, k) == 1          # f32 inputs
    assert L.flash_attn_bwd_grad16(*([A] * 8), NUL, *dims, q, k) == 1
    assert L.flash_attn_bwd_grad16(*([A] * 9), *dims, q, _lib.Layout(0, 64, 128)) == 1


def test_f16_dtype():
    # fp16 takes the 16-bit kernels: the same head dims and tilings as bf16
    assert fwd(dtype=2, D=96) == 2
    assert bwd(dtype=2, D=32) == 2
    assert dq_dvec(dtype=2, bq=64, bk=64) == 1
    for p in range(3):
        assert fa.flash_attn_default_tiles(2, 128, p) == fa.flash_attn_default_tiles(1, 128, p)
    assert fa.flash_attn_check_layout((64 * 4 * 128, 4 * 128, 128), 2, 64, 4, 128, 2) == 0
    assert fa.flash_attn_check_layout((4 * 64 * 130, 130, 64 * 130), 2, 64, 4, 128, 2) == 1
    assert fwd(dtype=3) == 1


def test_default_tiles():
    assert fa.flash_attn_default_tiles(1, 128, 0) == (128, 32)
    assert fa.flash_attn_default_tiles(1, 128, 1) == (32, 128)
    assert fa.flash_attn_default_tiles(1, 128, 2) == (128, 64)
    assert fa.flash_attn_default_tiles(0, 8, 0) == (64, 64)
    with pytest.raises(fa.FlashAttnError):
        fa.flash_attn_default_tiles(1, 80, 0)


# (strides (batch, row, head), B, T, heads, D, dtype, expected status)
LAYOUTS = [
    ((64 * 4 * 128, 4 * 128, 128), 2, 64, 4, 128, 1, 0),          # contiguous [B, T, h, D]
    ((4 * 64 * 128, 128, 64 * 128), 2, 64, 4, 128, 1, 0),         # [B, h, T, D] / [B*h, T, D]
    ((4 * 64 * 136, 136, 64 * 136), 2, 64, 4, 128, 1, 0),         # padded rows
    ((0, 4 * 128, 128), 1, 64, 4, 128, 1, 0),                     # batch stride unused at B = 1
    ((64 * 4 * 128, 4 * 128, 0), 2, 64, 1, 128, 1, 0),            # head stride unused at 1 head
    ((64 * 4 * 64, 4 * 64, 64), 2, 64, 4, 64, 0, 0),              # f32
    ((4 * 64 * 68, 68, 64 * 68), 2, 64, 4, 64, 0, 0),             # f32 rows of 68 (16 bytes)
    ((64 * 4 * 128, 4 * 128, 128), 2, 64, 4, 128, 7, 1),          # bad dtype
    ((64 * 4 * 128, -512, 128), 2, 64, 4, 128, 1, 1),             # negative stride
    ((4 * 64 * 64, 64, 64 * 64), 2, 64, 4, 128, 1, 1),            # rows shorter than D
    ((4 * 64 * 130, 130, 64 * 130), 2, 64, 4, 128, 1, 1),         # rows not 16-byte multiples
    ((4 * 64 * 66, 66, 64 * 66), 2, 64, 4, 64, 0, 1),             # f32 rows not 16-byte multiples
    ((64 * 128, 128, 128), 2, 64, 4, 128, 1, 1),                  # heads alias rows
    ((0, 4 * 128, 128), 2, 64, 4, 128, 1, 1),                     # batches alias
    ((64 * 4 * 128, 4 * 128, 64), 2, 64, 4, 128, 1, 1),           # heads overlap within a row
    ((1 << 33, 2048, 0), 1, 1 << 20, 1, 128, 1, 1),               # bf16 head span >= 2 GiB
    ((1 << 33, 2048, 0), 1, 1 << 20, 1, 128, 0, 0),               # same strides, f32: 64-bit
    ((64 * 4 * 128, 4 * 128, 128), 0, 64, 4, 128, 1, 1),          # B < 1
]


@pytest.mark.parametrize("strides,B,T,heads,D,dtype,code", LAYOUTS)
def test_layout_check(strides, B, T, heads, D, dtype, code):
    assert fa.flash_attn_check_layout(strides, B, T, heads, D, dtype) == code


def test_strided_entries_reject_before_launch():
    L = _lib.lib()
    dims = (1, 64, 64, 4, 2, 128, 0.125, 1, 0, 1, S0)   # B T Tk H HKV D scale causal window dtype
    good_q = _lib.Layout(64 * 4 * 128, 4 * 128, 128)
    good_k = _lib.Layout(64 * 2 * 128, 2 * 128, 128)
    bad = _lib.Layout(64 * 4 * 128, 64, 128)                       # rows shorter than D
    assert L.flash_attn_fwd_strided(A, A, A, A, A, *dims, bad, good_k) == 1
    assert L.flash_attn_fwd_strided(A, A, A, A, A, *dims, good_q, bad) == 1
    assert L.flash_attn_fwd_strided(A, NUL, A, A, A, *dims, good_q, good_k) == 1
    assert L.flash_attn_bwd_strided(*([A] * 9), *dims, bad, good_k) == 1
    assert L.flash_attn_bwd_strided(*([A] * 9), *dims, good_q, bad) == 1
    assert L.flash_attn_bwd_strided(*([A] * 8), MIS, *dims, good_q, good_k) == 1
    assert L.flash_attn_fwd_strided(A, A, A, A, A, 1, 64, 0, 4, 2, 128, 0.125, 1, 0, 1, S0,
                                    good_q, good_k) == 1                      # Tk < 1
    # the KV layout is checked with HKV heads: a head stride that aliases only at 4 heads
    kv2 = _lib.Layout(64 * 2 * 128, 2 * 128, 128)
    assert fa.flash_attn_check_layout((kv2.batch, kv2.row, kv2.head), 1, 64, 2, 128, 1) == 0


CLASS_SWEEP = [(T, bq, bk, c, w) for T in (1, 7, 64, 100, 129, 257, 300)
               for bq, bk in ((32, 32), (64, 16), (16, 64), (128, 64), (64, 128), (32, 64),
                              (16, 16), (5, 3))
               for c, w in ((True, 0), (True, 1), (True, 9), (True, 64), (False, 0),
                            (False, 5), (True, 1000))]


@pytest.mark.parametrize("T,bq,bk,causal,window", CLASS_SWEEP)
def test_device_classifier_matches_oracle(T, bq, bk, causal, window):
    cls = oracle.classify_blocks(T, bq, bk, causal, window)
    for i in range(cls.shape[0]):
        for j in range(cls.shape[1]):
            got, off = fa.flash_attn_block_class(T, bq, bk, causal, window, i, j)
            assert got == cls[i, j], (i, j)
            assert off == i * bq - j * bk
        lo, hi = fa.flash_attn_kv_block_range(T, bq, bk, causal, window, i)
        want = oracle.kv_block_range(i, bq, bk, T, causal, window)
        assert (lo, hi) == want, i


def test_device_partial_offsets_cycle_like_the_graphcore_walk():
    """Causal masked blocks met by the kernels' loops carry the offsets of the diagonal walk."""
    for bq, bk in ((64, 16), (32, 32), (16, 64), (128, 64)):
        T = 4 * np.lcm(bq, bk)
        seq = []
        for i in range(T // bq):
            lo, hi = fa.flash_attn_kv_block_range(T, bq, bk, True, 0, i)
            for j in range(lo, hi):
                c, off = fa.flash_attn_block_class(T, bq, bk, True, 0, i, j)
                if c == 2:
                    seq.append(off + 1)
        cyc = oracle.triu_offset_sequence(bq, bk)
        assert seq == [cyc[n % len(cyc)] for n in range(len(seq))]


RECT_SWEEP = [(Tq, Tk, bq, bk, c, w)
              for Tq, Tk in ((1, 7), (5, 64), (64, 5), (100, 129), (129, 100), (1, 300), (300, 17))
              for bq, bk in ((32, 32), (64, 16), (128, 64), (32, 64), (5, 3))
              for c, w in ((True, 0), (True, 9), (False, 0), (False, 5), (True, 1))]


@pytest.mark.parametrize("Tq,Tk,bq,bk,causal,window", RECT_SWEEP)
def test_rect_classifier_matches_oracle(Tq, Tk, bq, bk, causal, window):
    """T query rows against Tk keys: the device classifier and key-block ranges equal the
    oracle's brute force over the materialised mask."""
    cls = oracle.classify_blocks(Tq, bq, bk, causal, window, Tk)
    for i in range(cls.shape[0]):
        for j in range(cls.shape[1]):
            assert fa.flash_attn_block_class_qk(Tq, Tk, bq, bk, causal, window, i, j) == cls[i, j], (i, j)
        want = oracle.kv_block_range(i, bq, bk, Tq, causal, window, Tk)
        assert fa.flash_attn_kv_block_range_qk(Tq, Tk, bq, bk, causal, window, i) == want, i


def test_square_helpers_equal_rect_helpers_at_equal_lengths():
    for T, bq, bk, c, w in ((100, 32, 64, True, 0), (257, 128, 32, True, 7), (64, 16, 16, False, 3)):
        for i in range(-(-T // bq)):
            for j in range(-(-T // bk)):
                assert (fa.flash_attn_block_class(T, bq, bk, c, w, i, j)[0]
                        == fa.flash_attn_block_class_qk(T, T, bq, bk, c, w, i, j))


def rope(qk=A, f1=A, f2=A, oq=A, ok=A, st=8 * 128, sh=128, fst=128, tokens=4, heads=4, D=128,
         rd=128, paired=0, key_offset=0, dtype=1):
    return _lib.lib().flash_attn_qk_norm_rope(qk, st, sh, f1, f2, fst, oq, ok, tokens, heads, D,
                                              rd, paired, key_offset, dtype, S0)


@pytest.mark.parametrize("kw,code", [
    (dict(qk=NUL), 1), (dict(oq=MIS), 1), (dict(tokens=0), 1), (dict(heads=0), 1),
    (dict(D=96), 2), (dict(D=512), 2), (dict(rd=130), 1), (dict(rd=7), 1), (dict(rd=-2), 1),
    (dict(paired=1, key_offset=1), 1), (dict(paired=1, heads=3, st=6 * 128), 1),
    (dict(paired=2), 1), (dict(sh=64), 1), (dict(sh=132), 1), (dict(st=7 * 128), 1),
    (dict(fst=64), 1), (dict(fst=130), 1), (dict(paired=1, fst=128), 1), (dict(dtype=5), 1),
])
def test_rope_rejects_before_launch(kw, code):
    assert rope(**kw) == code

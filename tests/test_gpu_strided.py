"""Strided layouts through flash_attn_fwd_strided / flash_attn_bwd_strided (GPU): [B, H, T, D]
views, the thirds of a packed [3, B*H, T, D] QKV buffer, contiguous queries with [B, H, T, D]
keys, and rows padded with NaN.  The same kernels run with other address arithmetic only, so
every output must equal the contiguous path's bit for bit; each case is also checked against
the oracle.  T is ragged, so the rows past T of one head (which in [B, H, T, D] are the next
head's first rows) must still read as zeros."""
import math

import pytest
import torch

import oracle
import online_softmax_fwd_flash_amd as fa
from parity import compare, log, to_np
from workloads import make_inputs_like

pytestmark = pytest.mark.gpu

PAD = {"bf16": 8, "f16": 8, "f32": 4}   # extra elements per padded row (16 bytes)


def bhtd_view(x, pad=0):
    """x [B, T, h, D] (CPU) -> a [B, T, h, D] view of a [B, h, T, D + pad] cuda buffer whose
    pad columns hold NaN."""
    B, T, h, D = x.shape
    buf = torch.full((B, h, T, D + pad), float("nan"), dtype=x.dtype)
    buf[..., :D] = x.permute(0, 2, 1, 3)
    return buf.cuda().transpose(1, 2)[..., :D]


def packed_views(q, k, v):
    """Thirds of a packed [3, B*H, T, D] cuda buffer as [B, T, H, D] views."""
    B, T, H, D = q.shape
    buf = torch.empty((3, B * H, T, D), dtype=q.dtype)
    for i, x in enumerate((q, k, v)):
        buf[i] = x.permute(0, 2, 1, 3).reshape(B * H, T, D)
    buf = buf.cuda()
    return [buf[i].view(B, H, T, D).transpose(1, 2) for i in range(3)]


def make_views(kind, q, k, v, do, dtype):
    if kind == "bhtd":
        return bhtd_view(q), bhtd_view(k), bhtd_view(v), bhtd_view(do)
    if kind == "padded":
        p = PAD[dtype]
        return bhtd_view(q, p), bhtd_view(k, p), bhtd_view(v, p), bhtd_view(do, p)
    if kind == "packed":
        qv, kv, vv = packed_views(q, k, v)
        return qv, kv, vv, bhtd_view(do)
    if kind == "mixed":
        return q.cuda(), bhtd_view(k), bhtd_view(v), do.cuda()
    raise ValueError(kind)


CASES = [("bf16", 128), ("bf16", 64), ("f16", 128), ("f32", 64)]
KINDS = [("bhtd", 8, 2), ("padded", 8, 2), ("packed", 4, 4), ("mixed", 8, 2)]


@pytest.mark.parametrize("dtype,D", CASES)
@pytest.mark.parametrize("kind,H,HKV", KINDS)
@pytest.mark.parametrize("causal,window", [(True, 0), (False, 37)])
def test_strided_matches_contiguous_and_oracle(dtype, D, kind, H, HKV, causal, window):
    B, T = 2, 200
    scale = 1.0 / math.sqrt(D)
    log(f"strided {kind} {dtype} D={D} B={B} T={T} H={H} HKV={HKV} causal={causal} window={window}")
    q, k, v, do = make_inputs_like(B, T, H, HKV, D, dtype, 300 + D + H)
    qv, kv, vv, dov = make_views(kind, q, k, v, do, dtype)
    assert tuple(qv.shape) == (B, T, H, D) and tuple(kv.shape) == (B, T, HKV, D)

    o, lse = fa.flash_attn_fwd_strided(qv, kv, vv, causal=causal, window=window, scale=scale)
    # O comes back in q's strides; the backward wants dO in the same strides
    assert o.stride() == qv.stride()
    dq, dk, dv = fa.flash_attn_bwd_strided(qv, kv, vv, o, lse, dov, causal=causal,
                                           window=window, scale=scale)
    torch.cuda.synchronize()

    # the contiguous path on the same values
    qc, kc, vc, doc = (t.cuda() for t in (q, k, v, do))
    o_c, lse_c = fa.flash_attn_fwd(qc, kc, vc, causal=causal, window=window, scale=scale)
    dq_c, dk_c, dv_c = fa.flash_attn_bwd(qc, kc, vc, o_c, lse_c, doc, causal=causal,
                                         window=window, scale=scale)
    torch.cuda.synchronize()
    for name, got, want in (("O", o, o_c), ("L", lse, lse_c), ("dQ", dq, dq_c),
                            ("dK", dk, dk_c), ("dV", dv, dv_c)):
        assert torch.equal(got.contiguous(), want), f"{name} differs from the contiguous path"

    ref = oracle.attn_bwd(q, k, v, do, scale, causal, window)
    compare("O", to_np(o), ref["o"], dtype)
    compare("L", to_np(lse), ref["lse"], dtype)
    compare("dQ", to_np(dq), ref["dq"], dtype)
    compare("dK", to_np(dk), ref["dk"], dtype)
    compare("dV", to_np(dv), ref["dv"], dtype)

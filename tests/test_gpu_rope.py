"""QK RMS-norm + rotary prologue (GPU) against the fp64 oracle: bf16, fp16 and f32 rows of
64 and 128 elements, full and partial rotary tables, paired heads, key offset, and a QK
projection that is a slice of a wider QKV projection (token stride past the 2*heads rows)."""
import numpy as np
import pytest
import torch

import oracle
import online_softmax_fwd_flash_amd as fa
from parity import TOL, compare, log, to_np
from workloads import make_qk_packed, rotary_tables

pytestmark = pytest.mark.gpu

RTOL = dict(TOL)
RTOL["f32"] = dict(max_abs=1e-5, rel_l2=None)   # fp32 arithmetic on O(1) values


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("mode", ["plain", "partial_key_offset", "paired", "qkv_slice"])
def test_qk_norm_rope(dtype, D, mode):
    tokens, heads = 300, 4
    log(f"rope {dtype} D={D} {mode}")
    paired = mode == "paired"
    key_offset = mode == "partial_key_offset"
    rotary_dim = D // 2 if key_offset else D
    qk = make_qk_packed(tokens, heads, D, dtype, seed=900 + D)
    f1, f2 = rotary_tables(tokens, D, rotary_dim, pos0=11, halves=2 if paired else 1)
    if mode == "qkv_slice":
        # the QK part of a [tokens, (2*heads + 2) * D] QKV projection (two V heads after it)
        qkv = make_qk_packed(tokens, heads + 1, D, dtype, seed=901).reshape(tokens, -1)
        qkv[:, :2 * heads * D] = qk.reshape(tokens, -1)
        qkd = qkv.cuda()[:, :2 * heads * D].view(tokens, 2 * heads, D)
        assert qkd.stride(0) == (2 * heads + 2) * D
    else:
        qkd = qk.cuda()
    oq, ok = fa.flash_attn_qk_norm_rope(qkd, f1.cuda(), f2.cuda(), heads, rotary_dim,
                                        paired=paired, key_offset=key_offset)
    torch.cuda.synchronize()
    wq, wk = oracle.qk_norm_rope(qk, f1, f2, heads, rotary_dim, paired=paired,
                                 key_offset=key_offset)
    tol = RTOL[dtype]
    for name, got, want in (("Q", oq, wq), ("K", ok, wk)):
        g = to_np(got)
        assert g.shape == want.shape
        err = float(np.abs(g - want).max())
        assert err <= tol["max_abs"], f"{name}: max-abs {err:.3e}"
        if tol["rel_l2"] is not None:
            rel = float(np.linalg.norm(g - want) / np.linalg.norm(want))
            assert rel <= tol["rel_l2"], f"{name}: rel-L2 {rel:.3e}"

"""flash_attn_bwd_grad16 (GPU): dQ, dK, dV stored in the input's 16-bit type.  Each value must
be exactly the float32 gradient of flash_attn_bwd_strided rounded to nearest-even (torch's
conversion), and the tensors are held to the relative-L2 bound of their dtype against the
oracle (a 16-bit store of gradients up to ~9 cannot meet the absolute bound the float32
outputs meet)."""
import math

import numpy as np
import pytest
import torch

import oracle
import online_softmax_fwd_flash_amd as fa
from parity import TOL, log, to_np
from workloads import make_inputs_like

pytestmark = pytest.mark.gpu


def rel_l2(got, want):
    return float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-30))


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("bf16", 64), ("f16", 128)])
@pytest.mark.parametrize("layout", ["contiguous", "bhtd"])
@pytest.mark.parametrize("causal,window", [(True, 0), (False, 29)])
def test_grad16_is_rounded_fp32(dtype, D, layout, causal, window):
    B, T, H, HKV = 2, 260, 8, 2
    scale = 1.0 / math.sqrt(D)
    log(f"grad16 {dtype} D={D} {layout} causal={causal} window={window}")
    q, k, v, do = make_inputs_like(B, T, H, HKV, D, dtype, 500 + D)
    if layout == "contiguous":
        qv, kv, vv, dov = (t.cuda() for t in (q, k, v, do))
    else:
        qv, kv, vv, dov = (t.permute(0, 2, 1, 3).contiguous().cuda().transpose(1, 2)
                           for t in (q, k, v, do))
    o, lse = fa.flash_attn_fwd_strided(qv, kv, vv, causal=causal, window=window, scale=scale)
    g32 = fa.flash_attn_bwd_strided(qv, kv, vv, o, lse, dov, causal=causal, window=window,
                                    scale=scale)
    g16 = fa.flash_attn_bwd_grad16(qv, kv, vv, o, lse, dov, causal=causal, window=window,
                                   scale=scale)
    torch.cuda.synchronize()
    ref = oracle.attn_bwd(q, k, v, do, scale, causal, window)
    for name, a, b, r in zip(("dQ", "dK", "dV"), g16, g32, ("dq", "dk", "dv")):
        assert a.dtype == qv.dtype and a.stride() == b.stride()
        assert torch.equal(a, b.to(a.dtype)), f"{name}: not the rounded float32 gradient"
        err = rel_l2(to_np(a), ref[r])
        assert err <= TOL[dtype]["rel_l2"], f"{name}: rel-L2 {err:.3e}"

"""Each backward stage through its own C-ABI entry point vs the oracle (GPU): Dvec from the
preprocess, then dK/dV and dQ given the oracle-checked forward outputs; and the fused pass that
produces dQ and Dvec together."""
import math

import numpy as np
import pytest
import torch

import oracle
import online_softmax_fwd_flash_amd as fa
from parity import compare, gpu_fwd, log, to_np
from workloads import make_inputs_like

pytestmark = pytest.mark.gpu

CASES = [("f32", 64, (32, 32)), ("f32", 16, (64, 16)), ("bf16", 64, (0, 0)), ("bf16", 128, (0, 0)),
         ("f16", 128, (0, 0))]


def check_dvec(dvec, o, dod, ref, dtype):
    """Dvec is computed from the stored O (dtype precision), the oracle's from its fp64 O."""
    if dtype == "f32":
        compare("Dvec", to_np(dvec), ref["delta"], dtype)
        return
    # exact dot of the stored 16-bit O with dO, up to fp32 summation
    want = (to_np(o) * to_np(dod)).sum(-1).transpose(0, 2, 1)
    assert np.abs(to_np(dvec) - want).max() < 1e-4
    # and within the rounding of O (unit roundoff 2^-8 bf16, 2^-11 fp16) of the exact fp64 D
    u = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -11
    bound = u * np.abs(ref["o"] * to_np(dod)).sum(-1).transpose(0, 2, 1) + 1e-4
    assert (np.abs(to_np(dvec) - ref["delta"]) <= bound).all()


@pytest.mark.parametrize("dtype,D,tiles", CASES)
@pytest.mark.parametrize("causal,window", [(True, 0), (True, 9), (False, 0)])
def test_backward_stages(dtype, D, tiles, causal, window):
    B, T, H, HKV = 1, 160, 4, 2
    scale = 1.0 / math.sqrt(D)
    log(f"stages {dtype} D={D} tiles={tiles} causal={causal} window={window}")
    q, k, v, do = make_inputs_like(B, T, H, HKV, D, dtype, 90 + D)
    ref = oracle.attn_bwd(q, k, v, do, scale, causal, window)
    o, lse, (qd, kd, vd) = gpu_fwd(q, k, v, causal, window, scale, tiles)
    compare("O", to_np(o), ref["o"], dtype)
    dod = do.cuda()
    dvec = torch.full((B, H, T), float("nan"), device="cuda", dtype=torch.float32)
    fa.flash_attn_bwd_preprocess(o, dod, dvec)
    torch.cuda.synchronize()
    check_dvec(dvec, o, dod, ref, dtype)
    nan = float("nan")
    dk = torch.full(kd.shape, nan, device="cuda", dtype=torch.float32)
    dv = torch.full(kd.shape, nan, device="cuda", dtype=torch.float32)
    fa.flash_attn_bwd_dkdv(qd, kd, vd, dod, lse, dvec, causal=causal, window=window, scale=scale,
                           dk=dk, dv=dv, tiles=tiles)
    torch.cuda.synchronize()
    compare("dV", to_np(dv), ref["dv"], dtype)
    compare("dK", to_np(dk), ref["dk"], dtype)
    dq = torch.full(qd.shape, nan, device="cuda", dtype=torch.float32)
    fa.flash_attn_bwd_dq(qd, kd, vd, dod, lse, dvec, causal=causal, window=window, scale=scale,
                         dq=dq, tiles=tiles)
    torch.cuda.synchronize()
    compare("dQ", to_np(dq), ref["dq"], dtype)
    # dQ and Dvec from the one fused pass
    dq2 = torch.full(qd.shape, nan, device="cuda", dtype=torch.float32)
    dvec2 = torch.full((B, H, T), nan, device="cuda", dtype=torch.float32)
    fa.flash_attn_bwd_dq_dvec(qd, kd, vd, o, dod, lse, dvec=dvec2, causal=causal, window=window,
                              scale=scale, dq=dq2, tiles=tiles)
    torch.cuda.synchronize()
    check_dvec(dvec2, o, dod, ref, dtype)
    compare("dQ (fused Dvec)", to_np(dq2), ref["dq"], dtype)

"""flash_attn_bwd_noalloc (the backward for callers that cannot allocate) through the C ABI on
the GPU: its dQ, dK, dV equal flash_attn_bwd's bit for bit on the same inputs, and both meet
the oracle's tolerance.  Two calls in a row, the second on a smaller problem, so the second
call runs on a scratch array that still holds the first call's Dvec values; a problem larger
than the scratch is refused before anything is enqueued."""
import math

import pytest
import torch

import oracle
import online_softmax_fwd_flash_amd as fa
from online_softmax_fwd_flash_amd import _lib
from parity import compare, log, to_np
from workloads import make_inputs_like

pytestmark = pytest.mark.gpu

# (B, T, H, HKV, D, dtype, causal, window, seed): the second problem of each pair is smaller
PAIRS = [
    ((2, 300, 8, 2, 128, "bf16", True, 0, 41), (1, 130, 4, 1, 64, "bf16", True, 0, 42)),
    ((1, 257, 4, 2, 64, "f16", True, 33, 43), (1, 64, 2, 2, 64, "f16", False, 0, 44)),
    ((1, 200, 4, 4, 40, "f32", True, 0, 45), (1, 70, 2, 1, 16, "f32", True, 9, 46)),
]


def run_pair(case):
    B, T, H, HKV, D, dtype, causal, window, seed = case
    scale = 1.0 / math.sqrt(D)
    log(f"noalloc case B={B} T={T} H={H} HKV={HKV} D={D} {dtype} causal={causal} "
        f"window={window} seed={seed}")
    q, k, v, do = make_inputs_like(B, T, H, HKV, D, dtype, seed)
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, do))
    o, lse = fa.flash_attn_fwd(qd, kd, vd, causal=causal, window=window, scale=scale)
    nan = float("nan")
    outs = {}
    for name, fn in (("bwd", fa.flash_attn_bwd), ("noalloc", fa.flash_attn_bwd_noalloc)):
        dq = torch.full(qd.shape, nan, device="cuda", dtype=torch.float32)
        dk = torch.full(kd.shape, nan, device="cuda", dtype=torch.float32)
        dv = torch.full(kd.shape, nan, device="cuda", dtype=torch.float32)
        fn(qd, kd, vd, o, lse, dod, causal=causal, window=window, scale=scale, dq=dq, dk=dk,
           dv=dv)
        torch.cuda.synchronize()
        outs[name] = (dq, dk, dv)
    for a, b, what in zip(outs["bwd"], outs["noalloc"], ("dQ", "dK", "dV")):
        assert torch.equal(a, b), f"{what} differs between flash_attn_bwd and the no-alloc call"
    ref = oracle.attn_bwd(q, k, v, do, scale, causal, window)
    for t, name in zip(outs["noalloc"], ("dq", "dk", "dv")):
        compare(name, to_np(t), ref[name], dtype)


@pytest.mark.parametrize("pair", PAIRS, ids=lambda p: p[0][5])
def test_noalloc_matches_bwd_on_two_calls(pair):
    first, second = pair
    run_pair(first)
    run_pair(second)


def test_noalloc_refuses_more_than_its_scratch():
    # B * H * T one above the scratch: the call fails before touching the GPU buffers
    B, H, HKV, D = 1, 16, 2, 64
    T = _lib.FA_NOALLOC_MAX_DVEC // (B * H) + 1
    q = torch.empty(B, T, H, D, device="cuda", dtype=torch.bfloat16)
    k = torch.empty(B, T, HKV, D, device="cuda", dtype=torch.bfloat16)
    lse = torch.empty(B, H, T, device="cuda", dtype=torch.float32)
    dq = torch.empty(q.shape, device="cuda", dtype=torch.float32)
    dk = torch.empty(k.shape, device="cuda", dtype=torch.float32)
    with pytest.raises(fa.FlashAttnError) as e:
        fa.flash_attn_bwd_noalloc(q, k, k, q, lse, q, dq=dq, dk=dk, dv=dk.clone())
    assert e.value.code == _lib.FA_ERR_UNSUPPORTED

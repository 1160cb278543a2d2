"""Separate query and key lengths through flash_attn_fwd_strided / flash_attn_bwd_strided
(GPU) against the oracle: more keys than queries (a key prefix), more queries than keys
(under causal the first rows see no key: O = 0, L = 0, dQ = 0), one query (decode), with
causal, windowed and unmasked attention, GQA, every dtype."""
import math

import pytest
import torch

import oracle
import online_softmax_fwd_flash_amd as fa
from parity import compare, log, to_np
from workloads import make_inputs_like

pytestmark = pytest.mark.gpu

LENGTHS = [(100, 300), (300, 100), (1, 257), (129, 64), (64, 640)]
MASKS = [(True, 0), (True, 37), (False, 0), (False, 29)]


def inputs(B, Tq, Tk, H, HKV, D, dtype, seed):
    q, _, _, do = make_inputs_like(B, Tq, H, HKV, D, dtype, seed)
    _, k, v, _ = make_inputs_like(B, Tk, H, HKV, D, dtype, seed + 1)
    return q, k, v, do


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f16", 64), ("f32", 64)])
@pytest.mark.parametrize("Tq,Tk", LENGTHS)
@pytest.mark.parametrize("causal,window", MASKS)
def test_query_key_lengths(dtype, D, Tq, Tk, causal, window):
    B, H, HKV = 2, 8, 2
    scale = 1.0 / math.sqrt(D)
    log(f"qk {dtype} D={D} Tq={Tq} Tk={Tk} causal={causal} window={window}")
    q, k, v, do = inputs(B, Tq, Tk, H, HKV, D, dtype, 700 + Tq + Tk)
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, do))
    o, lse = fa.flash_attn_fwd_strided(qd, kd, vd, causal=causal, window=window, scale=scale)
    dq, dk, dv = fa.flash_attn_bwd_strided(qd, kd, vd, o, lse, dod, causal=causal,
                                           window=window, scale=scale)
    torch.cuda.synchronize()
    ref = oracle.attn_bwd(q, k, v, do, scale, causal, window)
    compare("O", to_np(o), ref["o"], dtype)
    compare("L", to_np(lse), ref["lse"], dtype)
    compare("dQ", to_np(dq), ref["dq"], dtype)
    compare("dK", to_np(dk), ref["dk"], dtype)
    compare("dV", to_np(dv), ref["dv"], dtype)
    if causal and Tq > Tk:
        # rows before the first key position: exactly zero
        n0 = Tq - Tk
        assert (o[:, :n0] == 0).all() and (lse[:, :, :n0] == 0).all() and (dq[:, :n0] == 0).all()

"""The hot path captured into a HIP graph (torch.cuda.CUDAGraph on ROCm) and replayed, as a
serving loop would run it: every replay gives the same bits as the eager calls, with other
GPU work and synchronisations between replays, and the eager result matches the oracle."""
import math

import pytest
import torch

import oracle
import online_softmax_fwd_flash_amd as fa
from parity import compare, log, to_np
from workloads import make_inputs_like

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("bf16", 64), ("f16", 128), ("f32", 64)])
def test_graph_replay_matches_eager(dtype, D):
    B, T, H, HKV = 1, 300, 8, 2
    causal, window = True, 0
    scale = 1.0 / math.sqrt(D)
    log(f"graph replay {dtype} D={D} B={B} T={T} H={H} HKV={HKV}")
    q, k, v, do = make_inputs_like(B, T, H, HKV, D, dtype, 11 + D)
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, do))
    f32 = torch.float32
    o = torch.empty_like(qd)
    lse = torch.empty(B, H, T, device="cuda", dtype=f32)
    dvec = torch.empty(B, H, T, device="cuda", dtype=f32)
    dq = torch.empty(qd.shape, device="cuda", dtype=f32)
    dk = torch.empty(kd.shape, device="cuda", dtype=f32)
    dv = torch.empty(kd.shape, device="cuda", dtype=f32)
    outs = {"O": o, "L": lse, "Dvec": dvec, "dQ": dq, "dK": dk, "dV": dv}
    kw = dict(causal=causal, window=window, scale=scale)

    def step():
        fa.flash_attn_fwd(qd, kd, vd, out=o, lse=lse, **kw)
        fa.flash_attn_bwd_dq_dvec(qd, kd, vd, o, dod, lse, dvec=dvec, dq=dq, **kw)
        fa.flash_attn_bwd_dkdv(qd, kd, vd, dod, lse, dvec, dk=dk, dv=dv, **kw)

    # eager (this also sets the kernels' LDS attributes before any capture)
    step()
    torch.cuda.synchronize()
    eager = {name: t.clone() for name, t in outs.items()}
    ref = oracle.attn_bwd(q, k, v, do, scale, causal, window)
    compare("O", to_np(o), ref["o"], dtype)
    compare("dQ", to_np(dq), ref["dq"], dtype)
    compare("dK", to_np(dk), ref["dk"], dtype)
    compare("dV", to_np(dv), ref["dv"], dtype)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in outs.values():
            t.fill_(float("nan"))   # eager work between replays; replay must rewrite all
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, t in outs.items():
            assert torch.equal(t, eager[name]), f"replay {rep}: {name} differs from eager"
    del graph


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f32", 64)])
def test_graph_of_public_entry_points(dtype, D):
    """flash_attn_fwd + flash_attn_bwd captured as they are: under capture the backward's Dvec
    workspace comes from stream-ordered allocation, which the graph records as memory nodes
    (the workspace cache is bypassed).  Every replay equals the eager call bit for bit."""
    B, T, H, HKV = 1, 300, 8, 2
    scale = 1.0 / math.sqrt(D)
    log(f"graph of public calls {dtype} D={D} B={B} T={T} H={H} HKV={HKV}")
    q, k, v, do = make_inputs_like(B, T, H, HKV, D, dtype, 31 + D)
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, do))
    f32 = torch.float32
    o = torch.empty_like(qd)
    lse = torch.empty(B, H, T, device="cuda", dtype=f32)
    dq = torch.empty(qd.shape, device="cuda", dtype=f32)
    dk = torch.empty(kd.shape, device="cuda", dtype=f32)
    dv = torch.empty(kd.shape, device="cuda", dtype=f32)
    outs = {"O": o, "L": lse, "dQ": dq, "dK": dk, "dV": dv}
    kw = dict(causal=True, window=0, scale=scale)

    def step():
        fa.flash_attn_fwd(qd, kd, vd, out=o, lse=lse, **kw)
        fa.flash_attn_bwd(qd, kd, vd, o, lse, dod, dq=dq, dk=dk, dv=dv, **kw)

    step()
    torch.cuda.synchronize()
    eager = {name: t.clone() for name, t in outs.items()}
    ref = oracle.attn_bwd(q, k, v, do, scale, True, 0)
    compare("dQ", to_np(dq), ref["dq"], dtype)
    compare("dK", to_np(dk), ref["dk"], dtype)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in outs.values():
            t.fill_(float("nan"))
        fa.flash_attn_bwd(qd, kd, vd, eager["O"], eager["L"], dod, **kw)   # eager call between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, t in outs.items():
            assert torch.equal(t, eager[name]), f"replay {rep}: {name} differs from eager"
    del graph

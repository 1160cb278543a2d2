"""flash_attn_bwd's workspace cache on the GPU.  A loop of calls on one stream does not hold the
host (it enqueues far faster than the GPU runs the calls); calls on several streams with no
host synchronisation between them, of growing sizes so that every rule of the cache is taken
(idle buffer, same stream, new slot, GPU-side wait, replacement of the smallest), give the
same bits as the no-alloc call made one at a time, which runs the same kernels."""
import math
import time

import pytest
import torch

import online_softmax_fwd_flash_amd as fa
from parity import log

pytestmark = pytest.mark.gpu


def _inputs(B, T, H, HKV, D, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    q = torch.randn(B, T, H, D, device="cuda", generator=g).bfloat16()
    k = torch.randn(B, T, HKV, D, device="cuda", generator=g).bfloat16()
    v = torch.randn(B, T, HKV, D, device="cuda", generator=g).bfloat16()
    do = torch.randn(B, T, H, D, device="cuda", generator=g).bfloat16()
    return q, k, v, do


def _grads(q, k):
    return (torch.empty(q.shape, device="cuda", dtype=torch.float32),
            torch.empty(k.shape, device="cuda", dtype=torch.float32),
            torch.empty(k.shape, device="cuda", dtype=torch.float32))


def test_loop_of_calls_does_not_hold_the_host():
    B, T, H, HKV, D = 2, 4096, 32, 8, 128
    log(f"workspace host timing B={B} T={T} H={H} HKV={HKV} D={D} bf16 causal")
    q, k, v, do = _inputs(B, T, H, HKV, D, 71)
    kw = dict(causal=True, window=0, scale=1 / math.sqrt(D))
    o, lse = fa.flash_attn_fwd(q, k, v, **kw)
    dq, dk, dv = _grads(q, k)
    fa.flash_attn_bwd(q, k, v, o, lse, do, dq=dq, dk=dk, dv=dv, **kw)
    torch.cuda.synchronize()
    n = 10
    t0 = time.perf_counter()
    for _ in range(n):
        fa.flash_attn_bwd(q, k, v, o, lse, do, dq=dq, dk=dk, dv=dv, **kw)
    t1 = time.perf_counter()
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    host, wall = t1 - t0, t2 - t0
    log(f"  {n} calls: host {host * 1e3:.3f} ms, wall {wall * 1e3:.3f} ms")
    assert host < 0.5 * wall, f"host held: enqueueing took {host:.4f} s of {wall:.4f} s"


def test_calls_on_several_streams_match_serial_calls():
    T, H, HKV, D = 4096, 16, 4, 64
    # B * H * T = 65536 B floats: B = 4i is i MiB of workspace, one cache granule per step
    sizes = [4, 8, 12, 16, 20]
    log(f"workspace streams T={T} H={H} HKV={HKV} D={D} bf16 causal, B in {sizes}")
    q, k, v, do = _inputs(max(sizes), T, H, HKV, D, 72)
    kw = dict(causal=True, window=0, scale=1 / math.sqrt(D))
    o, lse = fa.flash_attn_fwd(q, k, v, **kw)
    probs = [tuple(t[:B] for t in (q, k, v, o, lse, do)) for B in sizes]
    refs = []
    for p in probs:
        g = _grads(p[0], p[1])
        fa.flash_attn_bwd_noalloc(*p, dq=g[0], dk=g[1], dv=g[2], **kw)
        torch.cuda.synchronize()
        refs.append(g)
    streams = [torch.cuda.Stream() for _ in range(len(sizes))]
    # per stream: its own problem, then the first (smaller) problem again, no host syncs
    order = [(i, i) for i in range(len(sizes))] + [(i, 0) for i in range(len(sizes))]
    outs = [_grads(probs[pi][0], probs[pi][1]) for _, pi in order]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    for (si, pi), g in zip(order, outs):
        with torch.cuda.stream(streams[si]):
            fa.flash_attn_bwd(*probs[pi], dq=g[0], dk=g[1], dv=g[2], **kw)
    torch.cuda.synchronize()
    for (si, pi), g in zip(order, outs):
        for got, want, what in zip(g, refs[pi], ("dQ", "dK", "dV")):
            assert torch.equal(got, want), f"stream {si}, B={sizes[pi]}: {what} differs"

"""Checks that pin the fp64 oracle to facts fixed by the pages or by mathematics.

Each check takes an oracle-like module (attn_fwd, attn_bwd, attn_probs, group_of_head) and
raises AssertionError on failure, so the same checks run against the real oracle
(test_oracle_pins.py) and against copies with a planted mistake (test_oracle_mutants.py).
"""
import itertools
import math

import numpy as np
import torch

from workloads import make_inputs_like


def _tiny(B=1, T=9, H=4, HKV=2, D=5, seed=11):
    q, k, v, do = make_inputs_like(B, T, H, HKV, D, "f32", seed)
    return [t.double() for t in (q, k, v, do)]


MASKS = [(True, 0), (True, 3), (False, 0), (False, 4), (True, 1)]


def check_prob_rows(ora):
    """Every row of P is a probability distribution over its visible keys."""
    q, k, _, _ = _tiny()
    for causal, window in MASKS:
        P = ora.attn_probs(q, k, 0.7, causal, window)
        assert (P >= 0).all()
        assert np.allclose(P.sum(-1), 1.0, atol=1e-13, rtol=0)
        vis = np.ones((q.shape[1], q.shape[1]), bool)
        i, j = np.indices(vis.shape)
        if causal:
            vis &= j <= i
        if window:
            vis &= j >= i - window + 1
        assert (P[..., ~vis] == 0).all()


def check_causal_row0(ora):
    """Causal row 0 sees only key 0: O_0 = V_0 exactly and L_0 = S_00 (the diagonal is kept,
    forge flash_attention.metal forward kernel; FlashMetal keeps j <= i too)."""
    q, k, v, _ = _tiny()
    scale = 0.37
    for window in (0, 2):
        O, L = ora.attn_fwd(q, k, v, scale, True, window)
        B, T, H, D = q.shape
        HKV = k.shape[2]
        for h in range(H):
            g = h // (H // HKV)
            assert np.array_equal(O[:, 0, h, :], v[:, 0, g, :].numpy())
            s00 = scale * (q[:, 0, h, :] * k[:, 0, g, :]).sum(-1).numpy()
            assert np.allclose(L[:, h, 0], s00, atol=1e-14, rtol=0)


def check_equal_scores(ora):
    """With Q = 0 every visible score is 0: O_i is the mean of the visible V_j and
    L_i = ln(#visible keys of row i)."""
    _, k, v, _ = _tiny(T=12)
    q = torch.zeros(1, 12, 4, 5, dtype=torch.float64)
    T = 12
    for causal, window in MASKS:
        O, L = ora.attn_fwd(q, k, v, 1.3, causal, window)
        for i in range(T):
            hi = i if causal else T - 1
            lo = max(0, i - window + 1) if window else 0
            n = hi - lo + 1
            for h in range(4):
                g = h // 2
                want = v[0, lo:hi + 1, g, :].numpy().mean(0)
                assert np.allclose(O[0, i, h], want, atol=1e-14, rtol=0), (causal, window, i, h)
                assert abs(L[0, h, i] - math.log(n)) < 1e-14


def _masked_scores(q, k, scale, causal, window):
    B, T, H, D = q.shape
    rep = H // k.shape[2]
    kk = k.repeat_interleave(rep, dim=2)
    S = scale * torch.einsum("bihd,bjhd->bhij", q, kk)
    i = torch.arange(T)[:, None]
    j = torch.arange(T)[None, :]
    vis = torch.ones(T, T, dtype=torch.bool)
    if causal:
        vis &= j <= i
    if window:
        vis &= j >= i - window + 1
    return S, vis


def check_lse(ora):
    """L equals a direct log-sum-exp (torch.logsumexp) of the visible scores."""
    q, k, v, _ = _tiny()
    for causal, window in MASKS:
        _, L = ora.attn_fwd(q, k, v, 0.9, causal, window)
        S, vis = _masked_scores(q, k, 0.9, causal, window)
        want = torch.logsumexp(S.masked_fill(~vis, -math.inf), dim=-1).numpy()
        assert np.allclose(L, want, atol=1e-13, rtol=0)


def check_sdpa(ora, shapes=((2, 10, 4, 2, 6), (1, 17, 3, 3, 8), (1, 8, 8, 1, 4)),
               row_chunks=(1024, 3)):
    """O, dQ, dK, dV against CPU fp64 torch scaled_dot_product_attention with autograd
    (GQA through repeat_interleave, i.e. contiguous head groups; masks as explicit booleans).
    Row chunks of 3 make the oracle form most chunks against a strict sub-span of the keys
    (the causal bound, the window), so that path is held to the library routine too."""
    for (n, (B, T, H, HKV, D)), chunk in itertools.product(enumerate(shapes), row_chunks):
        q, k, v, do = make_inputs_like(B, T, H, HKV, D, "f32", 100 + n)
        q, k, v, do = (t.double() for t in (q, k, v, do))
        for causal, window in MASKS:
            scale = 1.0 / math.sqrt(D) * (1.5 if n == 1 else 1.0)
            res = ora.attn_bwd(q, k, v, do, scale, causal, window, row_chunk=chunk)
            O, L = ora.attn_fwd(q, k, v, scale, causal, window, row_chunk=chunk)
            qt = q.permute(0, 2, 1, 3).clone().requires_grad_()
            kt = k.permute(0, 2, 1, 3).clone().requires_grad_()
            vt = v.permute(0, 2, 1, 3).clone().requires_grad_()
            rep = H // HKV
            _, vis = _masked_scores(q, k, scale, causal, window)
            out = torch.nn.functional.scaled_dot_product_attention(
                qt, kt.repeat_interleave(rep, dim=1), vt.repeat_interleave(rep, dim=1),
                attn_mask=vis, scale=scale)
            out.backward(do.permute(0, 2, 1, 3))
            o_ref = out.detach().permute(0, 2, 1, 3).numpy()
            assert np.allclose(O, o_ref, atol=1e-12, rtol=0), ("O", causal, window)
            assert np.allclose(res["o"], o_ref, atol=1e-12, rtol=0)
            for name, t in (("dq", qt), ("dk", kt), ("dv", vt)):
                ref = t.grad.permute(0, 2, 1, 3).numpy()
                assert np.allclose(res[name], ref, atol=1e-11, rtol=0), (name, causal, window)


def check_finite_differences(ora):
    """Analytic gradients of sum(O * dO) against central differences (h = 1e-6, fp64)."""
    B, T, H, HKV, D = 1, 6, 2, 1, 4
    q, k, v, do = make_inputs_like(B, T, H, HKV, D, "f32", 7)
    q, k, v, do = (t.double().numpy() for t in (q, k, v, do))
    scale = 0.6
    h = 1e-6
    for causal, window in ((True, 0), (True, 3), (False, 0), (False, 2)):
        res = ora.attn_bwd(q, k, v, do, scale, causal, window)

        def loss(qq, kk, vv):
            O, _ = ora.attn_fwd(qq, kk, vv, scale, causal, window)
            return float((O * do).sum())

        for name, arr in (("dq", q), ("dk", k), ("dv", v)):
            num = np.zeros_like(arr)
            for idx in np.ndindex(arr.shape):
                a_p, a_m = arr.copy(), arr.copy()
                a_p[idx] += h
                a_m[idx] -= h
                args_p = [q, k, v]
                args_m = [q, k, v]
                pos = {"dq": 0, "dk": 1, "dv": 2}[name]
                args_p[pos], args_m[pos] = a_p, a_m
                num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
            err = np.abs(num - res[name]).max()
            assert err <= 1e-6 * max(1.0, np.abs(num).max()), (name, causal, window, err)


def check_invariants(ora):
    """Shift invariance of softmax: sum_j dK_j = 0.  Rows of P sum to 1:
    sum_j dV_j = sum over the group's heads and all rows of dO.  And D_i = sum_j P_ij dP_ij
    (the identity the forge page states for its D kernel)."""
    B, T, H, HKV, D = 2, 11, 4, 2, 6
    q, k, v, do = make_inputs_like(B, T, H, HKV, D, "f32", 21)
    q, k, v, do = (t.double() for t in (q, k, v, do))
    rep = H // HKV
    for causal, window in MASKS:
        res = ora.attn_bwd(q, k, v, do, 0.5, causal, window)
        assert np.abs(res["dk"].sum(axis=1)).max() < 1e-12
        dO = do.numpy()
        for g in range(HKV):
            want = dO[:, :, g * rep:(g + 1) * rep, :].sum(axis=(1, 2))
            assert np.allclose(res["dv"][:, :, g, :].sum(axis=1), want, atol=1e-12, rtol=0)
        P = ora.attn_probs(q, k, 0.5, causal, window)
        vv = v.numpy()
        for b in range(B):
            for hh in range(H):
                g = hh // rep
                dP = dO[b, :, hh, :] @ vv[b, :, g, :].T
                assert np.allclose((P[b, hh] * dP).sum(-1), res["delta"][b, hh], atol=1e-12)


def check_rect_decode(ora):
    """One query row against Tk keys (separate query and key lengths, teeny-kernels
    flash_attn2.rs flash_attention2_forward's n_ctx_q / n_ctx_k; the reading that the rows are
    the last positions): the row sits at position Tk - 1, so causal keeps every key and a
    window W the last min(W, Tk).  With Q = 0 every score is 0, so O is the mean of those V rows
    and L = ln(their count)."""
    Tk, H, HKV, D = 7, 4, 2, 5
    _, k, v, _ = _tiny(T=Tk, H=H, HKV=HKV, D=D, seed=23)
    q = torch.zeros(1, 1, H, D, dtype=torch.float64)
    for causal, window in MASKS:
        O, L = ora.attn_fwd(q, k, v, 0.9, causal, window)
        n = Tk if window <= 0 else min(window, Tk)
        for h in range(H):
            g = h // (H // HKV)
            want = v[0, Tk - n:, g, :].numpy().mean(axis=0)
            assert np.allclose(O[0, 0, h], want, atol=1e-14, rtol=0)
            assert abs(L[0, h, 0] - math.log(n)) < 1e-14


def check_rect_prefix(ora):
    """T query rows against Tk > T keys are the last T rows of the square Tk problem, whatever
    its first Tk - T query rows hold; with dO = 0 on those rows they add nothing to dK, dV, so
    the gradients agree too (the reading of separate lengths)."""
    Tk, T, H, HKV, D = 11, 4, 4, 2, 5
    q, k, v, do = _tiny(T=Tk, H=H, HKV=HKV, D=D, seed=21)
    do = do.clone()
    do[:, :Tk - T] = 0
    for causal, window in MASKS:
        O_sq, L_sq = ora.attn_fwd(q, k, v, 0.6, causal, window)
        O, L = ora.attn_fwd(q[:, Tk - T:], k, v, 0.6, causal, window)
        assert np.allclose(O, O_sq[:, Tk - T:], atol=1e-13, rtol=0)
        assert np.allclose(L, L_sq[:, :, Tk - T:], atol=1e-13, rtol=0)


def check_rect_prefix_grads(ora):
    Tk, T, H, HKV, D = 11, 4, 4, 2, 5
    q, k, v, do = _tiny(T=Tk, H=H, HKV=HKV, D=D, seed=21)
    do = do.clone()
    do[:, :Tk - T] = 0
    for causal, window in MASKS:
        sq = ora.attn_bwd(q, k, v, do, 0.6, causal, window)
        rc = ora.attn_bwd(q[:, Tk - T:], k, v, do[:, Tk - T:], 0.6, causal, window)
        assert np.allclose(rc["dq"], sq["dq"][:, Tk - T:], atol=1e-13, rtol=0)
        assert np.allclose(rc["dk"], sq["dk"], atol=1e-13, rtol=0)
        assert np.allclose(rc["dv"], sq["dv"], atol=1e-13, rtol=0)


def check_rect_more_queries(ora):
    """T > Tk: under causal the first T - Tk rows sit before the first key and see nothing
    (O = 0, L = 0, as for any row without a visible key) and the rest are the square Tk
    problem's rows; without causal every row sees all keys (window: a lower bound)."""
    T, Tk, H, HKV, D = 10, 6, 4, 2, 5
    q, _, _, _ = _tiny(T=T, H=H, HKV=HKV, D=D, seed=25)
    _, k, v, _ = _tiny(T=Tk, H=H, HKV=HKV, D=D, seed=26)
    for window in (0, 3):
        O, L = ora.attn_fwd(q, k, v, 0.8, True, window)
        assert (O[:, :T - Tk] == 0).all() and (L[:, :, :T - Tk] == 0).all()
        O_sq, L_sq = ora.attn_fwd(q[:, T - Tk:], k, v, 0.8, True, window)
        assert np.allclose(O[:, T - Tk:], O_sq, atol=1e-13, rtol=0)
        assert np.allclose(L[:, :, T - Tk:], L_sq, atol=1e-13, rtol=0)
    O, L = ora.attn_fwd(q, k, v, 0.8, False, 0)
    P = ora.attn_probs(q, k, 0.8, False, 0)
    assert (P > 0).all()


ALL_FORWARD = [check_prob_rows, check_causal_row0, check_equal_scores, check_lse,
               check_rect_decode, check_rect_prefix, check_rect_more_queries]
ALL_BACKWARD = [check_sdpa, check_finite_differences, check_invariants, check_rect_prefix_grads]

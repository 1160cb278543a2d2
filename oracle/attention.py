"""fp64 reference for exact scaled-dot-product attention with causal / sliding-window masks and
grouped-query heads.  TEST INFRASTRUCTURE ONLY (see the package docstring).

Everything is the plain definition, materialised: the score matrix of a (batch, head) is
formed (in chunks of query rows, which are independent), masked, soft-maxed and multiplied by
V.  Each chunk of rows is formed against the span of keys that some row of the chunk sees:
every key outside that span is masked for every row of the chunk, so it would add exactly zero
to each sum over visible keys that the definition takes.  There is no online softmax here, no
tiling of the key axis and no recomputation trick; those belong to the method under test, not
to the oracle.

Sources (web pages, cited by title and section):
  * forge "flash_attention.metal" (S.-P. Boucher), header comment and the forward kernel
    flash_attn_fwd: layouts Q/O [B,T,H,D], K/V [B,T,HKV,D], L [B,H,T]; GQA head map
    h -> h / (H/HKV); scale multiplies q.k; causal keeps keys j <= i; the window keeps the W
    keys ending at the query (self included, 0 = off) and adds only a lower bound; a row with
    no visible key gets O = 0 and L = 0; L = m + ln(l) in natural-log units.
  * forge "flash_attention.metal", backward section and the three backward kernels:
    D_i = dO_i . O_i, P recomputed from L, dS = P (dP - D), dQ and dK carry one factor of scale,
    dK and dV sum over the query heads of a KV group.
  * teeny-kernels "flash_attn2.rs", backward dQ and dK/dV doc comments: the same formulas.
  * Graphcore "flash_attention_qkv_packed.cpp", flashAttentionQKVPackedGrad: D = rowsum(O * dO),
    dV += P^T dO, dP = dO V^T, dS = P (dP - D), dQ += dS K, dK += dS^T Q.
  * teeny-kernels "flash_attn2.rs", flash_attention2_forward: separate query and key lengths
    (n_ctx_q, n_ctx_k).  No page states a causal rule for them.  Reading taken here: the T
    query rows are the last T of the Tk key positions (row i sits at position i + Tk - T, as
    after a cached key prefix), and the causal and window rules apply to that position.
"""
import numpy as np


def _f64(x):
    """Exact float64 copy of a numpy array or a (CPU) torch tensor of any float dtype."""
    if hasattr(x, "detach"):
        x = x.detach().cpu()
        if str(x.dtype) != "torch.float64":
            x = x.float()          # bf16/f16 -> f32 is exact
        x = x.numpy()
    return np.asarray(x, dtype=np.float64)


def group_of_head(h, H, HKV):
    """KV head that query head h reads: heads are grouped contiguously, rep = H/HKV per group
    (forge flash_attention.metal, forward kernel's hkv computation)."""
    return h // (H // HKV)


def visible_mask(T, causal, window, rows=None, Tk=None):
    """Boolean [len(rows), Tk] matrix: True where query row i may attend to key j.

    Query row i sits at key position p = i + Tk - T (p = i when Tk = T, the default).  Causal
    keeps j <= p (the diagonal is kept).  A window W > 0 keeps j >= p - W + 1, i.e. the W keys
    ending at the query, self included; without causal it is a lower bound only.
    """
    Tk = T if Tk is None else Tk
    i = np.arange(T)[:, None] if rows is None else np.asarray(rows)[:, None]
    p = i + (Tk - T)
    j = np.arange(Tk)[None, :]
    vis = np.ones((i.shape[0], Tk), dtype=bool)
    if causal:
        vis &= j <= p
    if window > 0:
        vis &= j >= p - window + 1
    return vis


def _key_span(vis):
    """Slice of the keys that at least one row of the boolean mask `vis` sees (empty when no
    row sees any)."""
    seen = np.flatnonzero(vis.any(axis=0))
    return slice(0, 0) if seen.size == 0 else slice(int(seen[0]), int(seen[-1]) + 1)


def _softmax_rows(S, vis):
    """Masked row softmax of S (fp64).  Returns P, m, l; rows with no visible key give P=0,
    m=0, l=0."""
    Sm = np.where(vis, S, -np.inf)
    any_vis = vis.any(axis=1)
    m = np.where(any_vis, Sm.max(axis=1, initial=-np.inf), 0.0)
    E = np.where(vis, np.exp(Sm - m[:, None]), 0.0)
    l = E.sum(axis=1)
    P = np.divide(E, l[:, None], out=np.zeros_like(E), where=l[:, None] > 0)
    return P, m, l


def _check_shapes(q, k, v=None):
    """(B, T, Tk, H, HKV, D) of q [B,T,H,D] and k, v [B,Tk,HKV,D]."""
    B, T, H, D = q.shape
    Bk, Tk, HKV, Dk = k.shape
    if (Bk, Dk) != (B, D) or H % HKV != 0:
        raise ValueError(f"bad shapes q{q.shape} k{k.shape}")
    if v is not None and v.shape != k.shape:
        raise ValueError(f"bad shapes k{k.shape} v{v.shape}")
    return B, T, Tk, H, HKV, D


def attn_probs(q, k, scale, causal, window):
    """Full probability tensor P [B,H,T,Tk] in fp64 (small inputs only)."""
    q, k = _f64(q), _f64(k)
    B, T, Tk, H, HKV, D = _check_shapes(q, k)
    vis = visible_mask(T, causal, window, Tk=Tk)
    P = np.zeros((B, H, T, Tk))
    for b in range(B):
        for h in range(H):
            g = group_of_head(h, H, HKV)
            S = scale * (q[b, :, h, :] @ k[b, :, g, :].T)
            P[b, h] = _softmax_rows(S, vis)[0]
    return P


def attn_fwd(q, k, v, scale, causal, window, row_chunk=1024, pairs=None):
    """Forward: O [B,T,H,D] and L [B,H,T], both fp64.

    O_i = sum_j P_ij V_j with P the masked softmax of S = scale * Q K^T;  L_i = m_i + ln(l_i)
    with m_i the row max and l_i the sum of exp(S_ij - m_i) over visible keys (natural log).
    `pairs` optionally restricts the work to a list of (b, h); other entries are left NaN.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, T, Tk, H, HKV, D = _check_shapes(q, k, v)
    O = np.full((B, T, H, D), np.nan)
    L = np.full((B, H, T), np.nan)
    todo = [(b, h) for b in range(B) for h in range(H)] if pairs is None else pairs
    for b, h in todo:
        g = group_of_head(h, H, HKV)
        for r0 in range(0, T, row_chunk):
            rows = np.arange(r0, min(T, r0 + row_chunk))
            vis = visible_mask(T, causal, window, rows, Tk)
            keys = _key_span(vis)
            S = scale * (q[b, rows, h, :] @ k[b, keys, g, :].T)
            P, m, l = _softmax_rows(S, vis[:, keys])
            O[b, rows, h, :] = P @ v[b, keys, g, :]
            L[b, h, rows] = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), 0.0)
    return O, L


def attn_fwd_rows(q, k, v, scale, causal, window, triples):
    """O rows and L values for a list of (b, h, i) triples, each computed on its own."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, T, Tk, H, HKV, D = _check_shapes(q, k, v)
    out_o = np.zeros((len(triples), D))
    out_l = np.zeros(len(triples))
    for n, (b, h, i) in enumerate(triples):
        g = group_of_head(h, H, HKV)
        S = scale * (q[b, i, h, :][None, :] @ k[b, :, g, :].T)
        P, m, l = _softmax_rows(S, visible_mask(T, causal, window, [i], Tk))
        out_o[n] = (P @ v[b, :, g, :])[0]
        out_l[n] = m[0] + np.log(l[0]) if l[0] > 0 else 0.0
    return out_o, out_l


def attn_bwd(q, k, v, do, scale, causal, window, row_chunk=1024, groups=None):
    """Backward of the loss sum(O * dO).  Returns dict with dq, dk, dv (fp64) and the oracle's
    own O, L, D.  `groups` optionally restricts to a list of (b, g) KV groups (the query heads
    of a group are the only ones that touch its dK/dV); other entries are left NaN.

    D_i = dO_i . O_i;  dP = dO V^T;  dS = P * (dP - D);  dQ = scale dS K;
    dK_j = scale sum_{h in group} sum_i dS_ij Q_i;  dV_j = sum_{h in group} sum_i P_ij dO_i.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, T, Tk, H, HKV, D = _check_shapes(q, k, v)
    if do.shape != q.shape:
        raise ValueError("dO must have the shape of Q")
    rep = H // HKV
    dq = np.full(q.shape, np.nan)
    dk = np.full(k.shape, np.nan)
    dv = np.full(v.shape, np.nan)
    O = np.full(q.shape, np.nan)
    L = np.full((B, H, T), np.nan)
    Dv = np.full((B, H, T), np.nan)
    todo = [(b, g) for b in range(B) for g in range(HKV)] if groups is None else groups
    for b, g in todo:
        dk[b, :, g, :] = 0.0
        dv[b, :, g, :] = 0.0
        Kg, Vg = k[b, :, g, :], v[b, :, g, :]
        for h in range(g * rep, (g + 1) * rep):
            for r0 in range(0, T, row_chunk):
                rows = np.arange(r0, min(T, r0 + row_chunk))
                vis = visible_mask(T, causal, window, rows, Tk)
                keys = _key_span(vis)
                Qc, dOc = q[b, rows, h, :], do[b, rows, h, :]
                Kc, Vc = Kg[keys], Vg[keys]
                S = scale * (Qc @ Kc.T)
                P, m, l = _softmax_rows(S, vis[:, keys])
                Oc = P @ Vc
                Dc = (dOc * Oc).sum(axis=1)
                dP = dOc @ Vc.T
                dS = P * (dP - Dc[:, None])
                dq[b, rows, h, :] = scale * (dS @ Kc)
                dk[b, keys, g, :] += scale * (dS.T @ Qc)
                dv[b, keys, g, :] += P.T @ dOc
                O[b, rows, h, :] = Oc
                L[b, h, rows] = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), 0.0)
                Dv[b, h, rows] = Dc
    return {"dq": dq, "dk": dk, "dv": dv, "o": O, "lse": L, "delta": Dv}

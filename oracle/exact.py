"""Exact (unquantized) attention forward and backward in float64.

Test infrastructure only.  This is the plain definition of what the SageBwd
path approximates: softmax attention with scale 1/sqrt(d) ("Attention Is All
You Need", listed under "Builds on" on the SageBwd page), the causal mask
keeping key j <= query i (top-left aligned, equal query and key lengths), and
the FlashAttention-2 backward formulas (FlashAttention-2, also under "Builds
on"):

    S = Q K^T / sqrt(d),  P = softmax_rows(S),  O = P V,  LSE_i = log sum_j exp S_ij
    dV = P^T dO,  dP = dO V^T,  Delta_i = sum_c dO_ic O_ic,
    dS = P * (dP - Delta),  dQ = dS K / sqrt(d),  dK = dS^T Q / sqrt(d)

With ``qk_norm`` the attention runs on QK-normalized queries and keys (the
SageBwd abstract, insight (i), calls QK-norm necessary for stable training at
many tokens per step): every token row of Q and of K is divided by its root
mean square, x_n = x / sqrt(mean_c x^2 + 1e-6) (unit gain), and the gradients
are carried back through it: with r = 1/sqrt(mean_c x^2 + 1e-6),
dx = r (dx_n - x_n mean_c(dx_n x_n)).

All functions take one head: arrays of shape [N, d], any float dtype (cast to
float64).  ``*_bh`` wrappers loop over [B, H, N, d].
"""
from __future__ import annotations

import numpy as np


QK_NORM_EPS = 1e-6


def qk_norm(x):
    """Row-wise QK-norm of one head: (x_n, r) with r = 1/sqrt(mean_c x^2 + eps)
    and x_n = x r."""
    x = np.asarray(x, np.float64)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=1) + QK_NORM_EPS)
    return x * r[:, None], r


def qk_norm_bwd(dxn, xn, r):
    """Gradient through qk_norm: dx = r (dx_n - x_n mean_c(dx_n x_n)).  From
    dx_n_i/dx_j = r delta_ij - r^3 x_i x_j / d."""
    dxn = np.asarray(dxn, np.float64)
    xn = np.asarray(xn, np.float64)
    return np.asarray(r, np.float64)[:, None] * (dxn - xn * np.mean(dxn * xn, axis=1, keepdims=True))


def _mask(nq: int, nk: int, causal: bool) -> np.ndarray:
    """True where the score is kept."""
    if not causal:
        return np.ones((nq, nk), dtype=bool)
    i = np.arange(nq)[:, None]
    j = np.arange(nk)[None, :]
    return j <= i


def scores(q, k, causal: bool, scale: float | None = None) -> np.ndarray:
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    d = q.shape[-1]
    sc = 1.0 / np.sqrt(d) if scale is None else scale
    s = (q @ k.T) * sc
    return np.where(_mask(q.shape[0], k.shape[0], causal), s, -np.inf)


def fwd(q, k, v, causal: bool, qk_norm: bool = False):
    """Return (O [N,d], LSE [N]) in float64 (dense softmax)."""
    if qk_norm:
        q, k = globals()["qk_norm"](q)[0], globals()["qk_norm"](k)[0]
    s = scores(q, k, causal)
    m = np.max(s, axis=1, keepdims=True)
    e = np.exp(s - m)
    l = np.sum(e, axis=1, keepdims=True)
    p = e / l
    o = p @ np.asarray(v, np.float64)
    lse = (m + np.log(l))[:, 0]
    return o, lse


def probs(q, k, causal: bool):
    s = scores(q, k, causal)
    m = np.max(s, axis=1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=1, keepdims=True)


def fwd_online(q, k, v, causal: bool, block: int = 16):
    """Blockwise online-softmax forward (FlashAttention-2 style running max
    and rescaling).  A second, independent formulation of ``fwd`` used to pin
    it; not used elsewhere."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    n, d = q.shape
    nk = k.shape[0]
    sc = 1.0 / np.sqrt(d)
    o = np.zeros((n, v.shape[1]))
    lse = np.zeros(n)
    for i in range(n):
        m_run = -np.inf
        l_run = 0.0
        acc = np.zeros(v.shape[1])
        for j0 in range(0, nk, block):
            j1 = min(nk, j0 + block)
            srow = (k[j0:j1] @ q[i]) * sc
            keep = np.ones(j1 - j0, bool) if not causal else (np.arange(j0, j1) <= i)
            if not keep.any():
                continue
            srow = np.where(keep, srow, -np.inf)
            m_new = max(m_run, float(np.max(srow)))
            alpha = np.exp(m_run - m_new) if np.isfinite(m_run) else 0.0
            e = np.exp(srow - m_new)
            l_run = l_run * alpha + float(np.sum(e))
            acc = acc * alpha + e @ v[j0:j1]
            m_run = m_new
        o[i] = acc / l_run
        lse[i] = m_run + np.log(l_run)
    return o, lse


def bwd(q, k, v, do, causal: bool, o=None, qk_norm: bool = False):
    """Return (dQ, dK, dV) in float64.  ``o`` (if given) is the forward output
    used for Delta = rowsum(dO * O); by default the exact forward output."""
    if qk_norm:
        qn, rq = globals()["qk_norm"](q)
        kn, rk = globals()["qk_norm"](k)
        dqn, dkn, dv = bwd(qn, kn, v, do, causal, o)
        return qk_norm_bwd(dqn, qn, rq), qk_norm_bwd(dkn, kn, rk), dv
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    do = np.asarray(do, np.float64)
    d = q.shape[-1]
    sc = 1.0 / np.sqrt(d)
    p = probs(q, k, causal)
    if o is None:
        o = p @ v
    o = np.asarray(o, np.float64)
    dv = p.T @ do
    dp = do @ v.T
    delta = np.sum(do * o, axis=1, keepdims=True)
    ds = p * (dp - delta)
    dq = (ds @ k) * sc
    dk = (ds.T @ q) * sc
    return dq, dk, dv


def dscores(q, k, v, do, causal: bool):
    """dS = P * (dP - Delta) with the exact forward output (for invariant pins)."""
    q = np.asarray(q, np.float64)
    p = probs(q, k, causal)
    o = p @ np.asarray(v, np.float64)
    dp = np.asarray(do, np.float64) @ np.asarray(v, np.float64).T
    delta = np.sum(np.asarray(do, np.float64) * o, axis=1, keepdims=True)
    return p * (dp - delta)


def sampled(q, k, v, do, causal: bool, qrows, krows, chunk: int = 512, qk_norm: bool = False):
    """The same quantities as ``fwd``/``bwd`` for long sequences, for a sample
    of query rows (O, LSE, dQ) and key rows (dK, dV), in row chunks so that the
    N x N matrices are never held at once.  Delta uses the exact O."""
    if qk_norm:
        qn, rq = globals()["qk_norm"](q)
        kn, rk = globals()["qk_norm"](k)
        o_s, lse_s, dq_s, dk_s, dv_s = sampled(qn, kn, v, do, causal, qrows, krows, chunk)
        qrows, krows = np.asarray(qrows), np.asarray(krows)
        return (o_s, lse_s, qk_norm_bwd(dq_s, qn[qrows], rq[qrows]), qk_norm_bwd(dk_s, kn[krows], rk[krows]), dv_s)
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    do = np.asarray(do, np.float64)
    n, d = q.shape
    sc = 1.0 / np.sqrt(d)
    qrows = np.asarray(qrows)
    krows = np.asarray(krows)
    o_s = np.zeros((qrows.size, d))
    lse_s = np.zeros(qrows.size)
    dq_s = np.zeros((qrows.size, d))
    dk_s = np.zeros((krows.size, d))
    dv_s = np.zeros((krows.size, d))
    pos = {int(r): i for i, r in enumerate(qrows)}
    cols = np.arange(n)
    for r0 in range(0, n, chunk):
        rows = np.arange(r0, min(n, r0 + chunk))
        s = (q[rows] @ k.T) * sc
        if causal:
            s = np.where(cols[None, :] <= rows[:, None], s, -np.inf)
        m = np.max(s, axis=1, keepdims=True)
        e = np.exp(s - m)
        l = np.sum(e, axis=1, keepdims=True)
        p = e / l
        o = p @ v
        delta = np.sum(do[rows] * o, axis=1)
        pk = p[:, krows]
        dv_s += pk.T @ do[rows]
        dsk = pk * (do[rows] @ v[krows].T - delta[:, None])
        dk_s += (dsk.T @ q[rows]) * sc
        sel = [i for i, r in enumerate(rows) if int(r) in pos]
        if sel:
            sel = np.asarray(sel)
            dp = do[rows[sel]] @ v.T
            ds = p[sel] * (dp - delta[sel, None])
            idx = [pos[int(r)] for r in rows[sel]]
            dq_s[idx] = (ds @ k) * sc
            o_s[idx] = o[sel]
            lse_s[idx] = (m[sel, 0] + np.log(l[sel, 0]))
    return o_s, lse_s, dq_s, dk_s, dv_s


def fwd_bh(q, k, v, causal: bool, qk_norm: bool = False):
    B, H, N, d = q.shape
    o = np.zeros((B, H, N, d))
    lse = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            o[b, h], lse[b, h] = fwd(q[b, h], k[b, h], v[b, h], causal, qk_norm)
    return o, lse


def bwd_bh(q, k, v, do, causal: bool, o=None, qk_norm: bool = False):
    B, H, N, d = q.shape
    out = [np.zeros((B, H, N, d)) for _ in range(3)]
    for b in range(B):
        for h in range(H):
            r = bwd(q[b, h], k[b, h], v[b, h], do[b, h], causal, None if o is None else o[b, h], qk_norm)
            for x, y in zip(out, r):
                x[b, h] = y
    return tuple(out)

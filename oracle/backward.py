"""Gradients of softmax attention in float64 -- the definition the chunked
backward must meet.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

[RA], "pet project" steps 5-7: the ring forward is followed by a loss and a
backward pass, and the result is compared with full attention.  The pages give
no backward formulas; this is the plain calculus of O = softmax(S) V with
S = scale * Q K^T, one query row at a time:

    P  = softmax over the visible keys of the row      (masked pairs: P = 0)
    dV = P^T dO
    dP = dO V^T
    D  = rowsum(dO * O)                 (= rowsum(P * dP))
    dS = P * (dP - D)                   (the softmax Jacobian applied to dP)
    dQ = scale * dS K,   dK = scale * dS^T Q

With GQA a key/value head's gradients are the sums over the query heads that
read it.  A row with no visible key has P = 0 and contributes nothing.

Chunked (ring) form: split the keys into chunks j.  With the row's log-sum-exp
lse over ALL keys (what the forward returns), P_ij = exp(S_ij - lse_i) is the
full-row softmax restricted to chunk j, so every term above is a sum of
per-chunk-pair contributions: dQ_i = sum_j dQ_ij, dK_j = sum_i dK_ij, dV_j =
sum_i dV_ij, with D_i computed once from the final O_i.
"""
from __future__ import annotations

import numpy as np


def _visible(n_q, n_k, causal, q_pos0, k_pos0):
    if not causal:
        return np.ones((n_q, n_k), dtype=bool)
    return (k_pos0 + np.arange(n_k))[None, :] <= (q_pos0 + np.arange(n_q))[:, None]


def attention_bwd_fp64(q, k, v, do, scale: float = 1.0, causal: bool = False,
                       q_pos0: int = 0, k_pos0: int = 0):
    """(dQ, dK, dV) of O = attention(q, k, v) for the upstream gradient dO.

    q, do: [B, Hq, n_q, d]; k, v: [B, Hkv, n_k, d].  Returns float64 arrays of
    the same shapes as q, k, v.
    """
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    B, Hq, n_q, d = q.shape
    Hkv, n_k = k.shape[1], k.shape[2]
    group = Hq // Hkv
    vis = _visible(n_q, n_k, causal, q_pos0, k_pos0)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            g = h // group
            s = np.where(vis, scale * (q[b, h] @ k[b, g].T), -np.inf)
            any_vis = vis.any(axis=1)
            m = np.where(any_vis, s.max(axis=1, initial=-np.inf), 0.0)
            e = np.where(vis, np.exp(s - m[:, None]), 0.0)
            l = np.where(any_vis, e.sum(axis=1), 1.0)
            p = e / l[:, None]
            o = p @ v[b, g]
            dv[b, g] += p.T @ do[b, h]
            dp = do[b, h] @ v[b, g].T
            D = (do[b, h] * o).sum(axis=1)
            ds = p * (dp - D[:, None])
            dq[b, h] = scale * (ds @ k[b, g])
            dk[b, g] += scale * (ds.T @ q[b, h])
    return dq, dk, dv


def rowsum_do_o_fp64(do, o):
    """D = rowsum(dO * O) per query row: [B, H, n, d] x2 -> [B, H, n]."""
    return (np.asarray(do, dtype=np.float64) * np.asarray(o, dtype=np.float64)).sum(axis=-1)


def chunk_attention_bwd_fp64(q, k, v, do, lse, D, scale: float = 1.0, causal: bool = False,
                             q_pos0: int = 0, k_pos0: int = 0):
    """One chunk pair's contributions (dQ_ij, dK_ij, dV_ij), given the rows'
    full log-sum-exp ``lse`` and ``D`` ([B, Hq, n_q] each, natural log)."""
    q, k, v, do, lse, D = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do, lse, D))
    B, Hq, n_q, d = q.shape
    Hkv, n_k = k.shape[1], k.shape[2]
    group = Hq // Hkv
    vis = _visible(n_q, n_k, causal, q_pos0, k_pos0)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            g = h // group
            s = scale * (q[b, h] @ k[b, g].T)
            # rows with lse = -inf have no visible key anywhere: P = 0
            fin = np.isfinite(lse[b, h])
            p = np.where(vis & fin[:, None], np.exp(s - np.where(fin, lse[b, h], 0.0)[:, None]), 0.0)
            dv[b, g] += p.T @ do[b, h]
            dp = do[b, h] @ v[b, g].T
            ds = p * (dp - D[b, h][:, None])
            dq[b, h] = scale * (ds @ k[b, g])
            dk[b, g] += scale * (ds.T @ q[b, h])
    return dq, dk, dv

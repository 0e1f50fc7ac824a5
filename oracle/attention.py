"""Full softmax attention in float64 -- the definition chunked attention must meet.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

[RA] section 1 and section 2: self-attention for a token needs every other
token of the sequence, i.e. one softmax over the whole row of scores
q.k_u for all keys u.  [HF] "¿Por qué la paralelización de secuencias?": the
standard implementation materialises that L x L matrix of weights.  This
function computes exactly that definition, one query row at a time (rows are
grouped into blocks only to bound memory; every row always sees all of its
keys at once -- there is no key chunking here).

Readings where the pages are silent (each listed in the design notes):
* scale: logits are ``scale * (q . k)``; the pages' pseudocode uses scale 1.
* causal: a key at global position kp is visible to a query at global
  position qp iff kp <= qp.  Query row t of the chunk sits at q_pos0 + t, key
  u at k_pos0 + u.
* GQA: query head h reads key/value head h // (Hq // Hkv).
* a row with no visible key has output 0 and log-sum-exp -inf.
* lse is the natural-log log-sum-exp of the scaled logits over visible keys.
"""
from __future__ import annotations

import numpy as np


def attention_fp64(q, k, v, scale: float = 1.0, causal: bool = False,
                   q_pos0: int = 0, k_pos0: int = 0, row_block: int = 256):
    """Softmax attention over all keys.

    q: [B, Hq, n_q, d], k and v: [B, Hkv, n_k, d] (any real dtype; promoted to
    float64).  Returns (O [B, Hq, n_q, d], lse [B, Hq, n_q]) in float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, n_q, d = q.shape
    Bk, Hkv, n_k, dk = k.shape
    if Bk != B or dk != d or v.shape != k.shape:
        raise ValueError("q/k/v shapes disagree")
    if Hkv <= 0 or Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    group = Hq // Hkv
    O = np.zeros((B, Hq, n_q, d), dtype=np.float64)
    lse = np.full((B, Hq, n_q), -np.inf, dtype=np.float64)
    key_pos = k_pos0 + np.arange(n_k)
    for b in range(B):
        for h in range(Hq):
            g = h // group
            K = k[b, g]                      # [n_k, d]
            V = v[b, g]
            for r0 in range(0, n_q, row_block):
                r1 = min(n_q, r0 + row_block)
                s = scale * (q[b, h, r0:r1] @ K.T)          # [rows, n_k]
                if causal:
                    qp = q_pos0 + np.arange(r0, r1)
                    visible = key_pos[None, :] <= qp[:, None]
                else:
                    visible = np.ones(s.shape, dtype=bool)
                s = np.where(visible, s, -np.inf)
                any_vis = visible.any(axis=1)
                m = np.where(any_vis, s.max(axis=1, initial=-np.inf), 0.0)
                w = np.where(visible, np.exp(s - m[:, None]), 0.0)
                l = w.sum(axis=1)
                safe_l = np.where(any_vis, l, 1.0)
                O[b, h, r0:r1] = np.where(any_vis[:, None], (w @ V) / safe_l[:, None], 0.0)
                lse[b, h, r0:r1] = np.where(any_vis, m + np.log(safe_l), -np.inf)
    return O, lse


def unmasked_pairs(n_q: int, n_k: int, causal: bool, q_pos0: int = 0, k_pos0: int = 0) -> int:
    """Number of visible (query, key) pairs of one block, counted directly."""
    if not causal:
        return n_q * n_k
    tot = 0
    for t in range(n_q):
        # keys u with k_pos0 + u <= q_pos0 + t
        tot += max(0, min(n_k, q_pos0 + t - k_pos0 + 1))
    return tot


def attention_at_positions_fp64(q, k, v, q_pos, k_pos, scale: float = 1.0, row_block: int = 256):
    """Causal softmax attention with explicit global positions.

    Same definition as ``attention_fp64`` with ``causal=True``, for tokens whose
    positions are not one contiguous run: query row t sits at ``q_pos[t]``, key
    u at ``k_pos[u]``, and u is visible to t iff ``k_pos[u] <= q_pos[t]``.
    q: [B, Hq, n_q, d], k and v: [B, Hkv, n_k, d]; q_pos [n_q], k_pos [n_k].
    Returns (O [B, Hq, n_q, d], lse [B, Hq, n_q]) in float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    k_pos = np.asarray(k_pos, dtype=np.int64)
    B, Hq, n_q, d = q.shape
    Hkv, n_k = k.shape[1], k.shape[2]
    if q_pos.shape != (n_q,) or k_pos.shape != (n_k,):
        raise ValueError("one position per query row and per key")
    if Hkv <= 0 or Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    group = Hq // Hkv
    O = np.zeros((B, Hq, n_q, d), dtype=np.float64)
    lse = np.full((B, Hq, n_q), -np.inf, dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            g = h // group
            for r0 in range(0, n_q, row_block):
                r1 = min(n_q, r0 + row_block)
                s = scale * (q[b, h, r0:r1] @ k[b, g].T)
                visible = k_pos[None, :] <= q_pos[r0:r1, None]
                s = np.where(visible, s, -np.inf)
                any_vis = visible.any(axis=1)
                m = np.where(any_vis, s.max(axis=1, initial=-np.inf), 0.0)
                w = np.where(visible, np.exp(s - m[:, None]), 0.0)
                l = w.sum(axis=1)
                safe_l = np.where(any_vis, l, 1.0)
                O[b, h, r0:r1] = np.where(any_vis[:, None], (w @ v[b, g]) / safe_l[:, None], 0.0)
                lse[b, h, r0:r1] = np.where(any_vis, m + np.log(safe_l), -np.inf)
    return O, lse


def segment_ids(L: int, seg_starts) -> np.ndarray:
    """Sample index of every position 0..L-1 of a packed sequence whose samples
    start at the sorted positions ``seg_starts`` (the first must be 0)."""
    starts = np.asarray(seg_starts, dtype=np.int64)
    if starts.size == 0 or starts[0] != 0 or np.any(np.diff(starts) <= 0) or starts[-1] >= max(L, 1):
        raise ValueError("sample starts must be strictly increasing, begin at 0 and lie below L")
    ids = np.zeros(L, dtype=np.int64)
    for s in starts[1:]:
        ids[s:] += 1
    return ids


def attention_packed_fp64(q, k, v, seg_starts, scale: float = 1.0, row_block: int = 256):
    """Causal attention over a packed sequence: query t sees key u iff both lie
    in the same sample and u <= t.  q, k, v in natural order ([B, H, L, d],
    the same packing for every batch row)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, L, d = q.shape
    Hkv = k.shape[1]
    group = Hq // Hkv
    ids = segment_ids(L, seg_starts)
    O = np.zeros((B, Hq, L, d), dtype=np.float64)
    lse = np.full((B, Hq, L), -np.inf, dtype=np.float64)
    pos = np.arange(L)
    for b in range(B):
        for h in range(Hq):
            g = h // group
            for r0 in range(0, L, row_block):
                r1 = min(L, r0 + row_block)
                s = scale * (q[b, h, r0:r1] @ k[b, g].T)
                visible = (ids[None, :] == ids[r0:r1, None]) & (pos[None, :] <= pos[r0:r1, None])
                s = np.where(visible, s, -np.inf)
                m = s.max(axis=1)                        # every row sees at least itself
                w = np.where(visible, np.exp(s - m[:, None]), 0.0)
                l = w.sum(axis=1)
                O[b, h, r0:r1] = (w @ v[b, g]) / l[:, None]
                lse[b, h, r0:r1] = m + np.log(l)
    return O, lse

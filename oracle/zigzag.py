"""Zigzag assignment of sequence pieces to ring ranks, and the causal attention
of one rank's shard under it, in float64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

[UL], opening paragraph, names Ring/ZigZag among the context-parallel methods
without spelling it out.  Reading (the usual one): the sequence of L tokens is
cut into 2P equal pieces of c = L / (2P) tokens; rank r holds piece r and piece
2P - 1 - r, in that order, as its local shard of 2c tokens.  Attention itself
does not change -- every query attends, causally by global position, to every
key of the whole sequence; only which tokens sit on which rank changes.  Under
a causal mask the split evens out the work: a rank's early piece sees the
early pieces of ranks <= r, its late piece sees every early piece and the late
pieces of ranks >= r.
"""
from __future__ import annotations

import numpy as np

from .attention import attention_at_positions_fp64


def zigzag_positions(rank: int, P: int, c: int) -> np.ndarray:
    """Global positions of the 2c tokens of rank ``rank``'s shard, in shard order."""
    if not (0 <= rank < P) or c < 0:
        raise ValueError("need 0 <= rank < P and c >= 0")
    early = rank * c + np.arange(c, dtype=np.int64)
    late = (2 * P - 1 - rank) * c + np.arange(c, dtype=np.int64)
    return np.concatenate([early, late])


def zigzag_shard(x, P: int, axis: int = -2):
    """Natural-order sequence (along ``axis``) -> [P, ...] stack of the ranks'
    shards, each holding its two pieces along ``axis``."""
    x = np.asarray(x)
    L = x.shape[axis]
    if L % (2 * P):
        raise ValueError("sequence length must be a multiple of 2P")
    c = L // (2 * P)
    return np.stack([np.take(x, zigzag_positions(r, P, c), axis=axis) for r in range(P)])


def zigzag_attention_fp64(q_local, k_pool, v_pool, rank: int, scale: float = 1.0):
    """Causal attention of rank ``rank``'s shard.

    q_local [B, Hq, 2c, d]; k_pool, v_pool [P, B, Hkv, 2c, d] (every rank's
    shard in the zigzag layout).  Returns (O [B, Hq, 2c, d], lse [B, Hq, 2c]).
    """
    k_pool = np.asarray(k_pool)
    v_pool = np.asarray(v_pool)
    P, n = k_pool.shape[0], k_pool.shape[3]
    if n % 2 or np.asarray(q_local).shape[2] != n:
        raise ValueError("shards hold 2c tokens")
    c = n // 2
    k_all = np.concatenate([k_pool[j] for j in range(P)], axis=2)
    v_all = np.concatenate([v_pool[j] for j in range(P)], axis=2)
    k_pos = np.concatenate([zigzag_positions(j, P, c) for j in range(P)])
    return attention_at_positions_fp64(q_local, k_all, v_all, zigzag_positions(rank, P, c), k_pos, scale=scale)


def zigzag_block_classes(rank: int, P: int):
    """(query piece, key rank, key piece, class) for every piece pair a rank
    meets: "full" when the key piece lies before the query piece, "diagonal"
    when they are the same piece, "skip" when it lies after."""
    out = []
    for qa in (rank, 2 * P - 1 - rank):
        for j in range(P):
            for kb in (j, 2 * P - 1 - j):
                cls = "full" if kb < qa else ("diagonal" if kb == qa else "skip")
                out.append((qa, j, kb, cls))
    return out

"""Online-softmax (log-sum-exp) merge and the ring visit, in float64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

[RA] section 3 and section 5: each device keeps its query chunk and, over
P - 1 exchanges, sees every other device's key/value chunk; each chunk's
partial attention is folded into the running output by an online-softmax
rescale so that the end result equals one softmax over all keys.

The pages' printed pseudocode does not implement that intent (it reuses the
first chunk's weights for later chunks, normalises the first chunk twice,
overwrites the running max with a log-sum-exp of maxima, and its row
statistics do not broadcast).  This oracle follows the stated intent, not the
listing: the state per query row is a normalised partial output O and its
natural-log log-sum-exp ``lse`` (equivalent to the running max / normaliser /
unnormalised accumulator form).  Merging two partials A and B over disjoint
key sets:

    lse = log(exp(lse_A) + exp(lse_B))
    O   = exp(lse_A - lse) * O_A + exp(lse_B - lse) * O_B

evaluated with the larger lse factored out.  A partial over no visible key is
(O = 0, lse = -inf) and is the identity of the merge.
"""
from __future__ import annotations

import numpy as np

from .attention import attention_fp64


def lse_merge_fp64(o_a, lse_a, o_b, lse_b):
    """Merge two partial attentions over disjoint key sets.

    o_*: [..., d], lse_*: [...] (same leading shape).  Returns (O, lse).
    """
    o_a = np.asarray(o_a, dtype=np.float64)
    o_b = np.asarray(o_b, dtype=np.float64)
    lse_a = np.asarray(lse_a, dtype=np.float64)
    lse_b = np.asarray(lse_b, dtype=np.float64)
    M = np.maximum(lse_a, lse_b)
    empty = np.isneginf(M)                      # both partials empty
    Ms = np.where(empty, 0.0, M)
    wa = np.where(np.isneginf(lse_a), 0.0, np.exp(lse_a - Ms))
    wb = np.where(np.isneginf(lse_b), 0.0, np.exp(lse_b - Ms))
    tot = wa + wb
    safe = np.where(empty, 1.0, tot)
    lse = np.where(empty, -np.inf, Ms + np.log(safe))
    O = (wa / safe)[..., None] * o_a + (wb / safe)[..., None] * o_b
    O = np.where(empty[..., None], 0.0, O)
    return O, lse


def ring_visit_order(rank: int, P: int):
    """Chunks visited by virtual rank ``rank``: its own chunk first, then the
    chunk received from the previous device at each step, i.e. (rank - s) mod P
    for s = 0 .. P-1 ([RA] section 3: send to the next device, receive from
    the previous one)."""
    return [(rank - s) % P for s in range(P)]


def ring_attention_fp64(q_chunk, k_chunks, v_chunks, rank: int, scale: float = 1.0,
                        causal: bool = False):
    """Ring attention for one virtual rank, chunk by chunk with LSE merges.

    q_chunk: [B, Hq, n, d] -- the rank's query chunk (global positions
    rank*n .. rank*n + n - 1, the contiguous split of [RA] section 2).
    k_chunks, v_chunks: sequences of P chunks [B, Hkv, n, d]; chunk j holds
    keys j*n .. j*n + n - 1.
    """
    P = len(k_chunks)
    n = np.asarray(q_chunk).shape[2]
    O = None
    lse = None
    for j in ring_visit_order(rank, P):
        o_j, lse_j = attention_fp64(q_chunk, k_chunks[j], v_chunks[j], scale=scale,
                                    causal=causal, q_pos0=rank * n, k_pos0=j * n)
        if O is None:
            O, lse = o_j, lse_j
        else:
            O, lse = lse_merge_fp64(O, lse, o_j, lse_j)
    return O, lse

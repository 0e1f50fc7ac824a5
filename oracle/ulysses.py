"""Ulysses sequence<->head all-to-all as an explicit index copy.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

[UL]: before attention each of the P devices of the context-parallel group
holds QKV of its sequence part for all heads, [local_seqlen, global_heads,
head_dim]; an all_to_all turns this into the whole sequence for a subset of
heads, [global_seqlen, local_heads, head_dim]; after attention a second
all_to_all turns the output back.  The group size may not exceed the number
of query heads, and with GQA the key/value heads are copied up to the group
size.  [HF] "En qué se diferencia Ulysses SP de FSDP CP": the head count must
divide evenly over the participating GPUs.

Readings (the pages do not fix them):
* shard p holds tokens p*n .. p*n + n - 1 (n = L / P), the contiguous split of
  [RA] section 2;
* rank r receives the contiguous head group r*H/P .. (r+1)*H/P - 1, and its
  sequence is the P received pieces concatenated in source-rank order -- what
  an all_to_all split along the head axis delivers;
* GQA replication repeats each source head R = H_dst / H_src times in place
  (repeat-interleave): destination head j comes from source head j // R.  With
  H_dst = P >= H_kv, rank r gets KV head r * H_kv // P, the same group a query
  head of rank r maps to.

The copies move raw element bit patterns; the arrays are indexed explicitly
by the formulas above, one (rank, rank, head) triple at a time with the token
axis as a slice (no reshape/transpose tricks).
"""
from __future__ import annotations

import numpy as np


def check_ulysses_shapes(P: int, L: int, H_src: int, H_dst: int):
    if P <= 0 or L < 0 or H_src <= 0 or H_dst <= 0:
        raise ValueError("sizes must be positive")
    if L % P != 0:
        raise ValueError("sequence length must be divisible by the group size")
    if H_dst % P != 0:
        raise ValueError("head count must be divisible by the group size")
    if H_dst < P:
        raise ValueError("group size may not exceed the head count")
    if H_dst % H_src != 0:
        raise ValueError("destination heads must be a whole replication of the source heads")


def replicated_head_source(j: int, H_src: int, H_dst: int) -> int:
    """Source head of destination head j under repeat-interleave replication."""
    return j // (H_dst // H_src)


def seq_to_head_naive(src, P: int, H_dst: int | None = None):
    """src: [P, n, H_src, d] (shard p = tokens p*n ..).  Returns [P, L, H_dst/P, d]."""
    src = np.asarray(src)
    Ps, n, H_src, d = src.shape
    if Ps != P:
        raise ValueError("src must hold P shards")
    H_dst = H_src if H_dst is None else H_dst
    L = P * n
    check_ulysses_shapes(P, L, H_src, H_dst)
    Hl = H_dst // P
    dst = np.empty((P, L, Hl, d), dtype=src.dtype)
    for r in range(P):                 # destination rank
        for p in range(P):             # source rank
            for hl in range(Hl):       # local head on the destination
                j = r * Hl + hl        # global destination head
                # all n tokens t of source shard p land at p*n + t
                dst[r, p * n:(p + 1) * n, hl, :] = src[p, :, replicated_head_source(j, H_src, H_dst), :]
    return dst


def head_to_seq_naive(src, P: int):
    """src: [P, L, H/P, d] (rank r = heads r*H/P ..).  Returns [P, L/P, H, d]."""
    src = np.asarray(src)
    Ps, L, Hl, d = src.shape
    if Ps != P:
        raise ValueError("src must hold P shards")
    H = Hl * P
    check_ulysses_shapes(P, L, H, H)
    n = L // P
    dst = np.empty((P, n, H, d), dtype=src.dtype)
    for p in range(P):                 # destination rank (sequence shard)
        for r in range(P):             # source rank (head group)
            for hl in range(Hl):
                # tokens t = 0 .. n-1 of shard p sit at p*n + t on rank r
                dst[p, :, r * Hl + hl, :] = src[r, p * n:(p + 1) * n, hl, :]
    return dst

"""Seeded synthetic inputs shared by the HIP path's tests/bench and the CPU oracle.

This module only *draws* inputs: it holds none of the attention, merge or
layout arithmetic.  Both sides receive the same bit patterns from here:

* Q, K, V are drawn as float32 N(0, 1) from ``numpy.random.default_rng(seed)``
  (PCG64), in the order Q, K, V.  Where a workload puts the softmax scale
  ``d**-0.5`` on Q, Q is multiplied by it in float32 before rounding.
* bf16 tensors are the float32 draws rounded to nearest-even and kept as their
  raw 16-bit patterns (``uint16``); ``bf16_bits_to_f64`` decodes them exactly.
* Ulysses inputs are bf16 patterns of N(0, 1) draws, or "tag" patterns whose
  bits name the source element (including NaN/Inf/-0/subnormal patterns, so a
  layout copy that goes through float arithmetic would be caught).

The workloads mirror the pages' shapes: 128k-token sequences with
Llama-8B-like heads (32 query heads, 8 KV heads, d = 128) split over P = 8
sequence shards, plus a tiny fp32 four-way ring emulation like the pages'
four-worker "pet project" check (Ring Attention Q&A, aivaro.ru answer 425,
section "Пет-проект для закрепления").
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = [
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "bf16_bits_to_f64",
    "normal_f32",
    "AttnWorkload",
    "UlyssesWorkload",
    "WORKLOADS",
    "attention_inputs",
    "ulysses_input",
    "tag_pattern_u16",
    "tag_pattern_u32",
    "SPECIAL_BF16_PATTERNS",
]


# --------------------------------------------------------------------------
# bit-pattern helpers (input encoding only)
# --------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray, chunk: int = 1 << 24) -> np.ndarray:
    """Round float32 values to bfloat16 (round-to-nearest-even); return uint16 bits.

    NaNs stay NaN (quiet bit forced); overflow past the largest finite bf16
    rounds to +/-inf, as IEEE RNE does.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    xf = x.reshape(-1)
    of = out.reshape(-1)
    for s in range(0, xf.size, chunk):
        u = xf[s:s + chunk].view(np.uint32).astype(np.uint64)
        bias = ((u >> 16) & 1) + 0x7FFF
        r = ((u + bias) >> 16).astype(np.uint16)
        nan = np.isnan(xf[s:s + chunk])
        if nan.any():
            r[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
        of[s:s + chunk] = r
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float64."""
    return bf16_bits_to_f32(b).astype(np.float64)


def normal_f32(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(size=shape, dtype=np.float32)


# --------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class AttnWorkload:
    """A chunked-attention workload.

    layout "bhnd": Q is one query chunk [B, Hq, n_q, d]; K and V are a pool of
    P resident chunks [P][B, Hkv, n, d] (shard-major), as the ring sees them.
    layout "shd": one Ulysses head share, Q [S, Hq, d], K/V [S, Hkv, d].
    layout "zigzag": as "bhnd", but every shard of n tokens holds the two
    sequence pieces r and 2P-1-r of n/2 tokens each (the zigzag split).
    """
    name: str
    seed: int
    dtype: str          # "f32" or "bf16"
    B: int
    Hq: int
    Hkv: int
    d: int
    L: int              # full sequence length
    P: int              # number of sequence chunks (virtual ranks)
    causal: bool
    q_scaled: bool      # Q multiplied by d**-0.5 before rounding
    layout: str = "bhnd"
    ranks: tuple = ()   # query chunks exercised (empty = all P)

    @property
    def n(self) -> int:
        return self.L // self.P

    @property
    def query_ranks(self) -> tuple:
        return self.ranks if self.ranks else tuple(range(self.P))

    def unmasked_pairs(self) -> int:
        """(query, key) pairs that take part, summed over query ranks and heads."""
        n = self.n
        tot = 0
        for i in self.query_ranks:
            if self.layout == "shd":
                # a single share: one "chunk" of the full length
                tot += self.L * (self.L + 1) // 2 if self.causal else self.L * self.L
                continue
            if self.layout == "zigzag":
                # 2P-1 fully visible piece pairs and 2 diagonal ones per rank
                c = n // 2
                tot += (2 * self.P - 1) * c * c + c * (c + 1) if self.causal else n * self.L
                continue
            for j in range(self.P):
                if not self.causal or j < i:
                    tot += n * n
                elif j == i:
                    tot += n * (n + 1) // 2
        return tot * self.B * self.Hq

    def flops(self) -> int:
        """Algorithmic FLOPs: 2*d for q.k plus 2*d for p*v per unmasked pair."""
        return 4 * self.d * self.unmasked_pairs()


@dataclasses.dataclass(frozen=True)
class UlyssesWorkload:
    name: str
    seed: int
    P: int
    L: int
    H: int
    d: int
    elem_bytes: int = 2

    @property
    def n(self) -> int:
        return self.L // self.P

    def bytes_per_direction(self) -> int:
        # every element is read once and written once
        return 2 * self.P * self.n * self.H * self.d * self.elem_bytes


WORKLOADS = {
    # tiny fp32 four-way ring emulation, non-causal, raw N(0,1) Q (no 1/sqrt(d))
    "ring_f32_tiny": AttnWorkload("ring_f32_tiny", 1, "f32", 1, 4, 4, 64, 1024, 4,
                                  False, False),
    # bf16 non-causal chunked attention, 32k tokens as 8 chunks of 4096
    "ring_bf16_32k": AttnWorkload("ring_bf16_32k", 2, "bf16", 1, 32, 32, 128, 32768, 8,
                                  False, True),
    # one GPU's ring share at 128k, causal: rank 7 of 8, chunks of 16384
    "ring_bf16_128k_rank7_causal": AttnWorkload(
        "ring_bf16_128k_rank7_causal", 4, "bf16", 1, 32, 32, 128, 131072, 8,
        True, True, "bhnd", (7,)),
    # the whole causal 128k ring (all 8 ranks), contiguous chunks of 16384
    "ring_bf16_128k_causal": AttnWorkload(
        "ring_bf16_128k_causal", 4, "bf16", 1, 32, 32, 128, 131072, 8,
        True, True, "bhnd"),
    # the same ring with the zigzag split: rank r holds pieces r and 15-r of 8192
    "zigzag_bf16_128k_causal": AttnWorkload(
        "zigzag_bf16_128k_causal", 6, "bf16", 1, 32, 32, 128, 131072, 8,
        True, True, "zigzag"),
    # one GPU's Ulysses share: full 128k sequence, 4 query heads, 1 KV head
    "ulysses_share_gqa_128k_causal": AttnWorkload(
        "ulysses_share_gqa_128k_causal", 5, "bf16", 1, 4, 1, 128, 131072, 1,
        True, True, "shd"),
}

ULYSSES_WORKLOADS = {
    # 8 shards of [16384, 32, 128] bf16 <-> [131072, 4, 128]
    "ulysses_131k_32h": UlyssesWorkload("ulysses_131k_32h", 3, 8, 131072, 32, 128, 2),
}


def attention_inputs(w: AttnWorkload, *, L: int | None = None, P: int | None = None,
                     Hq: int | None = None, Hkv: int | None = None):
    """Draw Q, K, V for workload ``w`` (optionally at a reduced size).

    Returns a dict with
      "q": query chunk(s), "k"/"v": the resident KV pool,
    each as uint16 bf16 patterns (dtype "bf16") or float32 (dtype "f32").

    layout "bhnd": q has shape [len(ranks), B, Hq, n, d] (the query chunks of the
    exercised ranks, in rank order); k, v have shape [P, B, Hkv, n, d].
    layout "shd": q [L, Hq, d]; k, v [L, Hkv, d].
    """
    L = w.L if L is None else L
    P = w.P if P is None else P
    Hq = w.Hq if Hq is None else Hq
    Hkv = w.Hkv if Hkv is None else Hkv
    rng = np.random.default_rng(w.seed)
    d = w.d
    if w.layout == "shd":
        qs, ks = (L, Hq, d), (L, Hkv, d)
    else:
        n = L // P
        qs, ks = (P, w.B, Hq, n, d), (P, w.B, Hkv, n, d)
    q = normal_f32(rng, qs)
    if w.q_scaled:
        q *= np.float32(1.0 / math.sqrt(d))
    k = normal_f32(rng, ks)
    v = normal_f32(rng, ks)
    if w.layout == "bhnd" and w.ranks:
        q = np.ascontiguousarray(q[list(w.ranks)])
    if w.dtype == "bf16":
        return {"q": f32_to_bf16_bits(q), "k": f32_to_bf16_bits(k), "v": f32_to_bf16_bits(v)}
    return {"q": q, "k": k, "v": v}


def ulysses_input(w: UlyssesWorkload, *, L: int | None = None, H: int | None = None) -> np.ndarray:
    """P shards [P, L/P, H, d] of bf16 N(0,1) patterns (uint16)."""
    L = w.L if L is None else L
    H = w.H if H is None else H
    rng = np.random.default_rng(w.seed)
    x = normal_f32(rng, (w.P, L // w.P, H, w.d))
    return f32_to_bf16_bits(x)


# --------------------------------------------------------------------------
# scores far from zero with every key aligned to its query
# --------------------------------------------------------------------------
LOG2E_F32 = np.float32(1.4426950408889634)


def bf16_values_rounding_down_under_log2e(count: int = 8):
    """The `count` bf16 values in [0.25, 0.5) whose product with log2(e),
    taken in float32 and rounded to bf16, lands furthest below the exact
    product.  Returns (uint16 patterns, relative shift of that product)."""
    bits = (0x3E80 + np.arange(128)).astype(np.uint16)          # 0.25 * (1 + m/128)
    x = bf16_bits_to_f64(bits)
    scaled = bf16_bits_to_f64(f32_to_bf16_bits(bf16_bits_to_f32(bits) * LOG2E_F32))
    rel = (scaled - x * float(LOG2E_F32)) / (x * float(LOG2E_F32))
    order = np.argsort(rel, kind="stable")[:count]
    return bits[order], rel[order]


def aligned_score_inputs(B: int, H: int, nq: int, nk: int, d: int, seed: int,
                         top_nats=(10.0, 18.0)):
    """bf16 Q, K, V (uint16 patterns) whose scores (scale 1) all lie far above
    zero and move together under any per-element rescaling of Q.

    Every query element is one of the bf16 values in [0.25, 0.5) whose copy
    scaled by log2(e) and re-rounded to bf16 falls furthest below the exact
    product, so a computation that rescales Q and rounds it again shifts every
    score of a row in the same direction.  Keys are positive and aligned with
    the queries: key u of head h has elements a_h * s_u * (1 + 0.2 z), z ~
    N(0, 1) clipped to [-2, 2], with s_u = 1 for half the keys and 0.97 for
    the other half, and a_h chosen so that a row's largest score is about
    top_nats[0] .. top_nats[1] nats (spread over the heads).  The row sums of
    exp(score) then lie far above 1 but well inside float range.  V is
    N(0, 1)."""
    rng = np.random.default_rng(seed)
    vals, _ = bf16_values_rounding_down_under_log2e()
    q = vals[rng.integers(0, len(vals), size=(B, H, nq, d))]
    qmean = float(np.mean(bf16_bits_to_f64(vals)))
    tops = np.linspace(top_nats[0], top_nats[1], H) if H > 1 else np.array([top_nats[1]])
    a = (tops / (d * qmean * 1.2)).astype(np.float32)           # 1.2: the largest keys' noise gain
    z = np.clip(rng.standard_normal((B, H, nk, d), dtype=np.float32), -2.0, 2.0)
    s = np.where(np.arange(nk) % 2 == 0, np.float32(1.0), np.float32(0.97)).astype(np.float32)
    k = a[None, :, None, None] * s[None, None, :, None] * (np.float32(1.0) + np.float32(0.2) * z)
    v = rng.standard_normal((B, H, nk, d), dtype=np.float32)
    return q, f32_to_bf16_bits(k), f32_to_bf16_bits(v)


# 16-bit patterns that a value-based copy would not preserve:
# quiet NaN with payload, signalling NaN, +inf, -inf, -0, smallest subnormal,
# largest subnormal, negative NaN.
SPECIAL_BF16_PATTERNS = np.array(
    [0x7FC1, 0x7F81, 0x7F80, 0xFF80, 0x8000, 0x0001, 0x007F, 0xFFC3], dtype=np.uint16)


def tag_pattern_u16(shape, seed: int = 0) -> np.ndarray:
    """uint16 array whose value names its flat index (mod 2**16), salted with the
    special patterns above at seeded positions."""
    size = int(np.prod(shape))
    t = (np.arange(size, dtype=np.uint64) * 40503 + seed).astype(np.uint16)
    rng = np.random.default_rng(seed + 12345)
    m = min(size, max(len(SPECIAL_BF16_PATTERNS), size // 16))
    pos = rng.choice(size, size=m, replace=False) if size > 0 else np.zeros(0, np.int64)
    t[pos] = SPECIAL_BF16_PATTERNS[np.arange(m) % len(SPECIAL_BF16_PATTERNS)]
    return t.reshape(shape)


def tag_pattern_u32(shape) -> np.ndarray:
    """uint32 array holding each element's flat index (unique below 2**32)."""
    size = int(np.prod(shape))
    return np.arange(size, dtype=np.uint32).reshape(shape)


def device_attention_inputs(w: AttnWorkload, device="cuda"):
    """Q, K, V of workload ``w`` drawn directly on the GPU from torch's seeded
    generator (same shapes and distributions as ``attention_inputs``; used for
    timing at full size, where drawing on the host would dominate)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(w.seed)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    d = w.d
    if w.layout == "shd":
        qs, ks = (w.L, w.Hq, d), (w.L, w.Hkv, d)
    else:
        qs = (len(w.query_ranks), w.B, w.Hq, w.n, d)
        ks = (w.P, w.B, w.Hkv, w.n, d)
    q = torch.randn(qs, generator=g, device=device, dtype=torch.float32)
    if w.q_scaled:
        q *= 1.0 / math.sqrt(d)
    q = q.to(dt)
    k = torch.randn(ks, generator=g, device=device, dtype=torch.float32).to(dt)
    v = torch.randn(ks, generator=g, device=device, dtype=torch.float32).to(dt)
    return {"q": q, "k": k, "v": v}


def device_ulysses_input(w: UlyssesWorkload, device="cuda"):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(w.seed)
    return torch.randn((w.P, w.n, w.H, w.d), generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)

"""Pins for the CPU oracle: checks against facts other than the oracle itself.

Each ``pin_*`` takes an oracle package (the real ``oracle`` or a copy with a
planted mistake) and raises AssertionError when the oracle disagrees with
* brute-force pure-Python loops on tiny inputs,
* an independent library implementation (torch's CPU scaled_dot_product_attention
  in float64, scipy's softmax / logsumexp, numpy reshape/transpose),
* closed forms and hand-derived fixtures in ``tests/golden/``,
* algebraic identities of the log-sum-exp merge,
* the identity the method rests on: chunked, LSE-merged attention equals one
  softmax over all keys (Ring Attention Q&A, aivaro.ru answer 425, section 3 and
  the four-worker check of its "pet project").

``ALL_PINS`` lists them; ``tests/test_oracle_pins.py`` runs each against the
real oracle and ``tests/test_oracle_mutants.py`` checks that planted mistakes
fail at least one.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _arr(x):
    return np.array(x, dtype=object).astype(np.float64) if not isinstance(x, np.ndarray) else x


def _floats(x):
    return np.array(json.loads(json.dumps(x).replace('"-inf"', "-1e999")), dtype=np.float64)


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    fin = np.isfinite(b)
    assert np.array_equal(np.isneginf(a), np.isneginf(b)), f"{what}: -inf positions differ"
    assert np.array_equal(fin, np.isfinite(a)), f"{what}: finite positions differ"
    err = np.max(np.abs(a[fin] - b[fin])) if fin.any() else 0.0
    assert err <= tol, f"{what}: max abs err {err:g} > {tol:g}"


# ----------------------------------------------------------------------------
# attention
# ----------------------------------------------------------------------------
def _bruteforce(q, k, v, scale, causal, q_pos0, k_pos0):
    """Pure-Python loops with math.exp; the definition written out element by element."""
    B, Hq, nq, d = q.shape
    Hkv, nk = k.shape[1], k.shape[2]
    grp = Hq // Hkv
    O = np.zeros((B, Hq, nq, d))
    lse = np.full((B, Hq, nq), -np.inf)
    for b in range(B):
        for h in range(Hq):
            g = h // grp
            for t in range(nq):
                keys = [u for u in range(nk) if (not causal) or (k_pos0 + u <= q_pos0 + t)]
                if not keys:
                    continue
                s = {u: scale * sum(float(q[b, h, t, e]) * float(k[b, g, u, e]) for e in range(d))
                     for u in keys}
                mx = max(s.values())
                w = {u: math.exp(s[u] - mx) for u in keys}
                tot = sum(w.values())
                for e in range(d):
                    O[b, h, t, e] = sum(w[u] * float(v[b, g, u, e]) for u in keys) / tot
                lse[b, h, t] = mx + math.log(tot)
    return O, lse


_BF_CASES = [
    # B, Hq, Hkv, nq, nk, d, scale, causal, q_pos0, k_pos0, seed
    (1, 2, 2, 3, 5, 4, 1.0, False, 0, 0, 11),
    (2, 4, 2, 4, 6, 3, 0.7, False, 0, 0, 12),
    (1, 4, 1, 5, 5, 4, 1.3, True, 0, 0, 13),
    (1, 2, 1, 4, 7, 2, 0.5, True, 6, 3, 14),     # query chunk ahead of the key chunk
    (1, 2, 2, 4, 3, 2, 1.0, True, 0, 2, 15),     # first query rows see no key
    (1, 8, 2, 3, 4, 5, 0.9, False, 0, 0, 16),    # GQA 4:1
]


def _rand_case(c):
    B, Hq, Hkv, nq, nk, d, scale, causal, qp, kp, seed = c
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, nq, d))
    k = rng.standard_normal((B, Hkv, nk, d))
    v = rng.standard_normal((B, Hkv, nk, d))
    return q, k, v, scale, causal, qp, kp


def pin_attention_bruteforce(orc):
    for c in _BF_CASES:
        q, k, v, scale, causal, qp, kp = _rand_case(c)
        O, lse = orc.attention_fp64(q, k, v, scale=scale, causal=causal, q_pos0=qp, k_pos0=kp)
        Ob, lb = _bruteforce(q, k, v, scale, causal, qp, kp)
        _close(O, Ob, 1e-12, f"O vs brute force {c}")
        _close(lse, lb, 1e-12, f"lse vs brute force {c}")


def pin_attention_sdpa(orc):
    """torch's CPU scaled_dot_product_attention in float64 (own GQA handling)."""
    import torch
    import torch.nn.functional as F
    for c in _BF_CASES + [(1, 4, 2, 40, 70, 16, 0.25, True, 50, 0, 17),
                          (2, 6, 3, 33, 33, 8, 1.0, False, 0, 0, 18)]:
        q, k, v, scale, causal, qp, kp = _rand_case(c)
        O, lse = orc.attention_fp64(q, k, v, scale=scale, causal=causal, q_pos0=qp, k_pos0=kp)
        nq, nk = q.shape[2], k.shape[2]
        qt, kt, vt = (torch.from_numpy(np.ascontiguousarray(x)) for x in (q, k, v))
        mask = None
        if causal:
            mask = (kp + torch.arange(nk))[None, :] <= (qp + torch.arange(nq))[:, None]
        rows = mask.any(dim=1) if mask is not None else torch.ones(nq, dtype=torch.bool)
        ref = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale,
                                             enable_gqa=True)
        ref = torch.where(rows[None, None, :, None], ref, torch.zeros_like(ref))
        _close(O, ref.numpy(), 1e-12, f"O vs torch SDPA {c}")
        grp = q.shape[1] // k.shape[1]
        s = scale * torch.matmul(qt, kt.repeat_interleave(grp, dim=1).transpose(-1, -2))
        if mask is not None:
            s = s.masked_fill(~mask, float("-inf"))
        _close(lse, torch.logsumexp(s, dim=-1).numpy(), 1e-12, f"lse vs torch logsumexp {c}")


def pin_attention_closed_forms(orc):
    from scipy.special import logsumexp, softmax
    rng = np.random.default_rng(21)
    d, nk = 8, 6
    k = rng.standard_normal((1, 1, nk, d))
    v = rng.standard_normal((1, 1, nk, d))
    # zero queries: uniform weights -> mean of V, lse = ln n_k
    O, lse = orc.attention_fp64(np.zeros((1, 1, 3, d)), k, v, scale=0.8)
    _close(O, np.broadcast_to(v.mean(axis=2, keepdims=True), O.shape), 1e-14, "Q=0 mean")
    _close(lse, np.full(lse.shape, math.log(nk)), 1e-14, "Q=0 lse")
    # constant values: output is the constant whatever the weights
    q = rng.standard_normal((1, 1, 4, d))
    O, _ = orc.attention_fp64(q, k, np.full_like(v, 2.5), scale=1.1)
    _close(O, np.full(O.shape, 2.5), 1e-13, "V const")
    # one key: O = v0, lse = scaled score
    O, lse = orc.attention_fp64(q, k[:, :, :1], v[:, :, :1], scale=0.6)
    _close(O, np.broadcast_to(v[:, :, :1], O.shape), 1e-14, "n_k=1 O")
    _close(lse, 0.6 * (q @ k[:, :, :1].transpose(0, 1, 3, 2))[..., 0], 1e-13, "n_k=1 lse")
    # causal row 0 with aligned chunks sees only key 0
    O, lse = orc.attention_fp64(q, k, v, scale=1.0, causal=True, q_pos0=5, k_pos0=5)
    _close(O[:, :, 0], v[:, :, 0], 1e-14, "causal row0 O")
    _close(lse[:, :, 0], (q[:, :, 0] * k[:, :, 0]).sum(-1), 1e-13, "causal row0 lse")
    # V = identity (n_k <= d): output rows are the softmax probabilities themselves
    eye = np.zeros((1, 1, nk, d))
    eye[0, 0, np.arange(nk), np.arange(nk)] = 1.0
    O, lse = orc.attention_fp64(q, k, eye, scale=0.9)
    s = 0.9 * (q[0, 0] @ k[0, 0].T)
    _close(O[0, 0, :, :nk], softmax(s, axis=1), 1e-14, "V=I softmax")
    _close(O[0, 0, :, nk:], np.zeros((4, d - nk)), 0.0, "V=I zero tail")
    _close(lse[0, 0], logsumexp(s, axis=1), 1e-13, "V=I logsumexp")
    # every key hidden: O = 0, lse = -inf
    O, lse = orc.attention_fp64(q, k, v, causal=True, q_pos0=0, k_pos0=100)
    _close(O, np.zeros_like(O), 0.0, "masked O")
    assert np.isneginf(lse).all(), "masked lse must be -inf"


def pin_attention_hand_golden(orc):
    g = _load("softmax_hand.json")
    q, k, v = (np.array(g[x], dtype=np.float64) for x in ("q", "k", "v"))
    for key, kw in (("noncausal", dict(causal=False)),
                    ("causal_q0_k0", dict(causal=True, q_pos0=0, k_pos0=0)),
                    ("causal_q_behind_keys", dict(causal=True, q_pos0=0, k_pos0=1))):
        O, lse = orc.attention_fp64(q, k, v, scale=g["scale"], **kw)
        _close(O, _floats(g[key]["O"]), 1e-14, f"hand {key} O")
        _close(lse, _floats(g[key]["lse"]), 1e-14, f"hand {key} lse")
    # the same example read through GQA: 2 query heads share the single KV head
    q2 = np.concatenate([q, q[:, :, ::-1]], axis=1)
    O, lse = orc.attention_fp64(q2, k, v, scale=g["scale"])
    ref = _floats(g["noncausal"]["O"])
    _close(O[:, 1], ref[:, 0, ::-1], 1e-14, "hand GQA head 1")


def pin_unmasked_pairs(orc):
    for nq, nk, qp, kp in [(5, 5, 0, 0), (4, 7, 6, 3), (3, 4, 0, 2), (16, 16, 32, 0), (8, 8, 0, 20)]:
        want = sum(1 for t in range(nq) for u in range(nk) if kp + u <= qp + t)
        assert orc.unmasked_pairs(nq, nk, True, qp, kp) == want
        assert orc.unmasked_pairs(nq, nk, False, qp, kp) == nq * nk
    n = 16384
    assert orc.unmasked_pairs(n, n, True, 7 * n, 7 * n) == n * (n + 1) // 2


# ----------------------------------------------------------------------------
# merge and ring
# ----------------------------------------------------------------------------
def pin_merge_algebra(orc):
    rng = np.random.default_rng(31)
    o_a, o_b, o_c = (rng.standard_normal((3, 5, 4)) for _ in range(3))
    l_a, l_b, l_c = (rng.standard_normal((3, 5)) * 3 for _ in range(3))
    empty_o, empty_l = np.zeros_like(o_a), np.full_like(l_a, -np.inf)
    O, L = orc.lse_merge_fp64(o_a, l_a, empty_o, empty_l)
    _close(O, o_a, 1e-15, "merge identity O")
    _close(L, l_a, 1e-15, "merge identity lse")
    O, L = orc.lse_merge_fp64(empty_o, empty_l, o_b, l_b)
    _close(O, o_b, 1e-15, "merge left identity O")
    O, L = orc.lse_merge_fp64(o_a, l_a, o_a, l_a)
    _close(O, o_a, 1e-14, "merge self O")
    _close(L, l_a + math.log(2.0), 1e-14, "merge self lse")
    O1, L1 = orc.lse_merge_fp64(o_a, l_a, o_b, l_b)
    O2, L2 = orc.lse_merge_fp64(o_b, l_b, o_a, l_a)
    _close(O1, O2, 1e-15, "merge commutes O")
    _close(L1, L2, 0.0, "merge commutes lse")
    Oa, La = orc.lse_merge_fp64(*orc.lse_merge_fp64(o_a, l_a, o_b, l_b), o_c, l_c)
    Ob, Lb = orc.lse_merge_fp64(o_a, l_a, *orc.lse_merge_fp64(o_b, l_b, o_c, l_c))
    _close(Oa, Ob, 1e-13, "merge associates O")
    _close(La, Lb, 1e-13, "merge associates lse")
    O, L = orc.lse_merge_fp64(empty_o, empty_l, empty_o, empty_l)
    _close(O, empty_o, 0.0, "merge empty O")
    assert np.isneginf(L).all()
    # closed form: two single-key partials (v0, s0), (v1, s1) merge to a softmax over {s0, s1}
    s0, s1 = 0.3, -1.7
    v0, v1 = np.array([1.0, -2.0]), np.array([4.0, 0.5])
    O, L = orc.lse_merge_fp64(v0[None], np.array([s0]), v1[None], np.array([s1]))
    e0, e1 = math.exp(s0), math.exp(s1)
    _close(O[0], (e0 * v0 + e1 * v1) / (e0 + e1), 1e-15, "two-key merge O")
    _close(L[0], math.log(e0 + e1), 1e-15, "two-key merge lse")


_RING_CASES = [
    # P, n, B, Hq, Hkv, d, causal, scale, seed
    (1, 5, 1, 2, 2, 4, False, 1.0, 41),
    (2, 5, 1, 2, 1, 4, True, 0.5, 42),
    (3, 17, 2, 2, 2, 8, False, 0.3, 43),
    (4, 1, 1, 4, 2, 3, True, 1.0, 44),
    (4, 17, 1, 4, 4, 6, True, 0.4, 45),
    (4, 16, 1, 2, 2, 16, False, 1.0, 46),
]


def pin_ring_equals_full(orc):
    for P, n, B, Hq, Hkv, d, causal, scale, seed in _RING_CASES:
        rng = np.random.default_rng(seed)
        L = P * n
        q = rng.standard_normal((B, Hq, L, d))
        k = rng.standard_normal((B, Hkv, L, d)) * 2.0
        v = rng.standard_normal((B, Hkv, L, d))
        Of, lf = orc.attention_fp64(q, k, v, scale=scale, causal=causal)
        kc = [k[:, :, j * n:(j + 1) * n] for j in range(P)]
        vc = [v[:, :, j * n:(j + 1) * n] for j in range(P)]
        for i in range(P):
            O, lse = orc.ring_attention_fp64(q[:, :, i * n:(i + 1) * n], kc, vc, i, scale=scale,
                                             causal=causal)
            _close(O, Of[:, :, i * n:(i + 1) * n], 1e-12, f"ring O P={P} n={n} rank {i}")
            _close(lse, lf[:, :, i * n:(i + 1) * n], 1e-12, f"ring lse P={P} n={n} rank {i}")


def pin_ring_visit_order(orc):
    for P in range(1, 9):
        for i in range(P):
            order = orc.ring_visit_order(i, P)
            assert order[0] == i, "a rank starts with its own chunk"
            assert sorted(order) == list(range(P)), "every chunk visited exactly once"
            # step s receives what the previous rank held at step s-1
            for s in range(1, P):
                assert order[s] == orc.ring_visit_order((i - 1) % P, P)[s - 1]


# ----------------------------------------------------------------------------
# Ulysses
# ----------------------------------------------------------------------------
def pin_ulysses_hand_golden(orc):
    g = _load("ulysses_hand.json")
    for c in g["cases"]:
        src = np.array(c["src"], dtype=np.int64)
        want = np.array(c["dst"], dtype=np.int64)
        got = orc.seq_to_head_naive(src, g["P"], c["H_dst"])
        assert np.array_equal(got, want), f"hand case {c['H_src']}->{c['H_dst']}"
        if c["H_src"] == c["H_dst"]:
            assert np.array_equal(orc.head_to_seq_naive(want, g["P"]), src)


def pin_ulysses_library_form(orc):
    """Agreement with numpy's reshape/transpose statement of the all_to_all:
    [P, n, P, Hl, d] -> [P(rank), P(source), n, Hl, d]."""
    rng = np.random.default_rng(51)
    for P, n, H, d in [(2, 3, 4, 5), (4, 2, 8, 3), (3, 5, 6, 2), (8, 2, 8, 4), (1, 4, 3, 2)]:
        src = rng.integers(0, 1 << 16, size=(P, n, H, d), dtype=np.uint16)
        Hl = H // P
        lib = src.reshape(P, n, P, Hl, d).transpose(2, 0, 1, 3, 4).reshape(P, P * n, Hl, d)
        got = orc.seq_to_head_naive(src, P)
        assert np.array_equal(got, lib), f"seq->head vs transpose P={P}"
        back = orc.head_to_seq_naive(got, P)
        lib_back = got.reshape(P, P, n, Hl, d).transpose(1, 2, 0, 3, 4).reshape(P, n, H, d)
        assert np.array_equal(back, lib_back), f"head->seq vs transpose P={P}"


def pin_ulysses_roundtrip_tags(orc):
    from sequence_kv_chunk_amd.synth import tag_pattern_u16, tag_pattern_u32
    for P, n, H, d in [(2, 3, 2, 4), (4, 5, 8, 3), (8, 2, 16, 2), (1, 3, 2, 5)]:
        for src in (tag_pattern_u16((P, n, H, d), seed=P), tag_pattern_u32((P, n, H, d))):
            mid = orc.seq_to_head_naive(src, P)
            assert mid.shape == (P, P * n, H // P, d)
            assert np.array_equal(np.sort(mid.reshape(-1)), np.sort(src.reshape(-1))), "bijection"
            assert np.array_equal(orc.head_to_seq_naive(mid, P), src), "round trip"
            if P == 1:
                assert np.array_equal(mid.reshape(src.shape), src), "P=1 identity"
        # with unique tags, every output element names its source
        src = tag_pattern_u32((P, n, H, d))
        mid = orc.seq_to_head_naive(src, P)
        Hl = H // P
        for r in range(P):
            for s in range(P * n):
                for hl in range(Hl):
                    idx = int(mid[r, s, hl, 0])
                    p, t, h = idx // (n * H * d), (idx // (H * d)) % n, (idx // d) % H
                    assert (p * n + t, r * Hl + hl) == (s, h), "tag names its source"


def pin_ulysses_replication(orc):
    from sequence_kv_chunk_amd.synth import tag_pattern_u32
    for P, Hq, Hkv in [(8, 32, 8), (8, 32, 2), (8, 8, 1), (4, 8, 2), (2, 8, 4), (4, 4, 4)]:
        n, d = 3, 2
        H_dst = max(Hkv, P)
        src = tag_pattern_u32((P, n, Hkv, d))
        dst = orc.seq_to_head_naive(src, P, H_dst)
        Hl = H_dst // P
        head_of = (dst[..., 0] // d) % Hkv                   # [P, L, Hl]
        counts = np.bincount(head_of[:, 0, :].reshape(-1), minlength=Hkv)
        assert (counts == H_dst // Hkv).all(), "each KV head copied H_dst/H_kv times"
        # the KV head a rank holds is the group of every query head it holds
        for r in range(P):
            qheads = range(r * Hq // P, (r + 1) * Hq // P)
            kv_groups = sorted({h // (Hq // Hkv) for h in qheads})
            assert sorted(set(head_of[r, 0].tolist())) == kv_groups, f"P={P} Hkv={Hkv} rank {r}"


def pin_ulysses_limits(orc):
    src = np.zeros((4, 2, 8, 2), dtype=np.uint16)
    for bad in [lambda: orc.seq_to_head_naive(np.zeros((3, 2, 8, 2)), 3),       # 8 % 3
                lambda: orc.seq_to_head_naive(np.zeros((8, 2, 4, 2)), 8),       # P > H
                lambda: orc.seq_to_head_naive(src, 4, 12),                      # 12 % 8
                lambda: orc.check_ulysses_shapes(4, 10, 8, 8)]:                 # L % P
        try:
            bad()
        except ValueError:
            continue
        raise AssertionError("limit not enforced")


# ----------------------------------------------------------------------------
# attention at explicit positions, zigzag split
# ----------------------------------------------------------------------------
def _bruteforce_pos(q, k, v, q_pos, k_pos, scale):
    """Pure-Python loops: key u visible to query t iff k_pos[u] <= q_pos[t]."""
    B, Hq, nq, d = q.shape
    Hkv, nk = k.shape[1], k.shape[2]
    grp = Hq // Hkv
    O = np.zeros((B, Hq, nq, d))
    lse = np.full((B, Hq, nq), -np.inf)
    for b in range(B):
        for h in range(Hq):
            g = h // grp
            for t in range(nq):
                keys = [u for u in range(nk) if int(k_pos[u]) <= int(q_pos[t])]
                if not keys:
                    continue
                s = {u: scale * sum(float(q[b, h, t, e]) * float(k[b, g, u, e]) for e in range(d)) for u in keys}
                mx = max(s.values())
                w = {u: math.exp(s[u] - mx) for u in keys}
                tot = sum(w.values())
                for e in range(d):
                    O[b, h, t, e] = sum(w[u] * float(v[b, g, u, e]) for u in keys) / tot
                lse[b, h, t] = mx + math.log(tot)
    return O, lse


def pin_attention_at_positions(orc):
    rng = np.random.default_rng(31)
    for B, Hq, Hkv, nq, nk, d in [(1, 2, 1, 5, 7, 3), (2, 4, 2, 4, 6, 2)]:
        q = rng.standard_normal((B, Hq, nq, d))
        k = rng.standard_normal((B, Hkv, nk, d))
        v = rng.standard_normal((B, Hkv, nk, d))
        q_pos = rng.permutation(12)[:nq]
        k_pos = rng.permutation(12)[:nk]
        q_pos[0] = -1                                  # a query that sees no key
        O, lse = orc.attention_at_positions_fp64(q, k, v, q_pos, k_pos, scale=0.8)
        Ob, lb = _bruteforce_pos(q, k, v, q_pos, k_pos, 0.8)
        _close(O, Ob, 1e-12, "O at positions vs brute force")
        _close(lse, lb, 1e-12, "lse at positions vs brute force")
        # reordering the keys together with their positions changes nothing
        perm = rng.permutation(nk)
        O2, l2 = orc.attention_at_positions_fp64(q, k[:, :, perm], v[:, :, perm], q_pos, k_pos[perm], scale=0.8)
        _close(O2, O, 1e-12, "key order")
        _close(l2, lse, 1e-12, "key order lse")


def pin_zigzag_positions(orc):
    for P in range(1, 7):
        for c in (1, 3, 4):
            L = 2 * P * c
            allpos = np.concatenate([orc.zigzag_positions(r, P, c) for r in range(P)])
            assert sorted(allpos.tolist()) == list(range(L)), "every token on exactly one rank"
            for r in range(P):
                pos = orc.zigzag_positions(r, P, c)
                assert pos.shape == (2 * c,)
                # piece r then piece 2P-1-r, each a contiguous run of c tokens
                assert pos.tolist() == list(range(r * c, r * c + c)) + \
                    list(range((2 * P - 1 - r) * c, (2 * P - r) * c))
    # P = 1: the shard is the whole sequence in natural order
    assert orc.zigzag_positions(0, 1, 5).tolist() == list(range(10))
    x = np.arange(2 * 3 * 2 * 4).reshape(1, 2 * 3 * 2, 4)            # [1, L=12, 4], P=3, c=2
    sh = orc.zigzag_shard(x, 3, axis=1)
    assert sh.shape == (3, 1, 4, 4)
    assert sh[1, 0, :, 0].tolist() == [8, 12, 32, 36], "rank 1 holds tokens 2,3 and 8,9"


def pin_zigzag_equals_full(orc):
    """Every rank's zigzag shard result, put back in natural order, equals one
    causal softmax over the whole sequence (the contiguous definition)."""
    rng = np.random.default_rng(33)
    for P, c, B, Hq, Hkv, d, scale in [(1, 3, 1, 2, 1, 4, 1.0), (2, 2, 1, 2, 2, 3, 0.7),
                                       (3, 2, 2, 4, 2, 2, 1.2), (4, 1, 1, 2, 1, 3, 1.0)]:
        L = 2 * P * c
        q = rng.standard_normal((B, Hq, L, d))
        k = rng.standard_normal((B, Hkv, L, d)) * 1.5
        v = rng.standard_normal((B, Hkv, L, d))
        Of, lf = orc.attention_fp64(q, k, v, scale=scale, causal=True)
        kp = np.stack([k[:, :, [t for t in range(L) if (t // c) in (j, 2 * P - 1 - j)]] for j in range(P)])
        vp = np.stack([v[:, :, [t for t in range(L) if (t // c) in (j, 2 * P - 1 - j)]] for j in range(P)])
        for r in range(P):
            rows = [t for t in range(L) if (t // c) in (r, 2 * P - 1 - r)]
            O, lse = orc.zigzag_attention_fp64(q[:, :, rows], kp, vp, r, scale=scale)
            _close(O, Of[:, :, rows], 1e-12, f"zigzag O P={P} rank {r}")
            _close(lse, lf[:, :, rows], 1e-12, f"zigzag lse P={P} rank {r}")


def pin_zigzag_balance(orc):
    """Equal causal work on every rank: (2P-1) full piece pairs and 2 diagonal
    ones, i.e. 2P*c^2 + c visible pairs, counted directly from positions."""
    for P in range(1, 9):
        for c in (1, 2, 5):
            for r in range(P):
                cls = [x[3] for x in orc.zigzag_block_classes(r, P)]
                assert cls.count("full") == 2 * P - 1 and cls.count("diagonal") == 2
                assert cls.count("skip") == 4 * P - (2 * P - 1) - 2
                qp = orc.zigzag_positions(r, P, c)
                kp = np.concatenate([orc.zigzag_positions(j, P, c) for j in range(P)])
                pairs = int(np.sum(kp[None, :] <= qp[:, None]))
                assert pairs == 2 * P * c * c + c, (P, c, r, pairs)
                for qa, j, kb, cl in orc.zigzag_block_classes(r, P):
                    assert cl == ("full" if kb < qa else "diagonal" if kb == qa else "skip")
                    assert kb in (j, 2 * P - 1 - j) and qa in (r, 2 * P - 1 - r)


# ----------------------------------------------------------------------------
# backward
# ----------------------------------------------------------------------------
_BWD_CASES = [
    # B, Hq, Hkv, nq, nk, d, scale, causal, q_pos0, k_pos0, seed
    (1, 2, 1, 4, 5, 3, 0.8, False, 0, 0, 41),
    (1, 2, 2, 5, 5, 2, 1.1, True, 0, 0, 42),
    (2, 4, 2, 3, 6, 2, 1.0, True, 4, 2, 43),     # GQA, offset positions
    (1, 2, 1, 3, 4, 2, 1.0, True, 0, 2, 44),     # first row sees no key
]


def pin_backward_finite_differences(orc):
    """Central differences of L = sum(dO * O) through the (pinned) forward."""
    for c in _BWD_CASES:
        B, Hq, Hkv, nq, nk, d, scale, causal, qp, kp, seed = c
        rng = np.random.default_rng(seed)
        q = rng.standard_normal((B, Hq, nq, d))
        k = rng.standard_normal((B, Hkv, nk, d))
        v = rng.standard_normal((B, Hkv, nk, d))
        do = rng.standard_normal((B, Hq, nq, d))
        dq, dk, dv = orc.attention_bwd_fp64(q, k, v, do, scale=scale, causal=causal, q_pos0=qp, k_pos0=kp)

        def loss(q_, k_, v_):
            O, _ = orc.attention_fp64(q_, k_, v_, scale=scale, causal=causal, q_pos0=qp, k_pos0=kp)
            return float((O * do).sum())
        eps = 1e-6
        for name, x, g in (("dq", q, dq), ("dk", k, dk), ("dv", v, dv)):
            num = np.zeros_like(x)
            it = np.nditer(x, flags=["multi_index"])
            for _ in it:
                i = it.multi_index
                xp, xm = x.copy(), x.copy()
                xp[i] += eps
                xm[i] -= eps
                args_p = [q, k, v]
                args_m = [q, k, v]
                idx = {"dq": 0, "dk": 1, "dv": 2}[name]
                args_p[idx], args_m[idx] = xp, xm
                num[i] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            _close(g, num, 1e-6, f"{name} vs finite differences {c}")


def pin_backward_autograd(orc):
    """torch autograd in float64 on the CPU through its own attention."""
    import torch
    for c in _BWD_CASES + [(1, 4, 2, 17, 23, 8, 0.3, True, 10, 0, 45), (2, 2, 1, 9, 9, 4, 1.0, False, 0, 0, 46)]:
        B, Hq, Hkv, nq, nk, d, scale, causal, qp, kp, seed = c
        rng = np.random.default_rng(seed)
        q = rng.standard_normal((B, Hq, nq, d))
        k = rng.standard_normal((B, Hkv, nk, d))
        v = rng.standard_normal((B, Hkv, nk, d))
        do = rng.standard_normal((B, Hq, nq, d))
        dq, dk, dv = orc.attention_bwd_fp64(q, k, v, do, scale=scale, causal=causal, q_pos0=qp, k_pos0=kp)
        qt, kt, vt = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        grp = Hq // Hkv
        s = scale * torch.matmul(qt, kt.repeat_interleave(grp, dim=1).transpose(-1, -2))
        if causal:
            mask = (kp + torch.arange(nk))[None, :] <= (qp + torch.arange(nq))[:, None]
            s = s.masked_fill(~mask, float("-inf"))
            rows = mask.any(dim=1)
        else:
            rows = torch.ones(nq, dtype=torch.bool)
        p = torch.softmax(s, dim=-1)
        p = torch.where(rows[None, None, :, None], p, torch.zeros_like(p))     # empty rows: 0, not NaN
        o = torch.matmul(p, vt.repeat_interleave(grp, dim=1))
        (o * torch.tensor(do)).sum().backward()
        _close(dq, qt.grad.numpy(), 1e-12, f"dq vs autograd {c}")
        _close(dk, kt.grad.numpy(), 1e-12, f"dk vs autograd {c}")
        _close(dv, vt.grad.numpy(), 1e-12, f"dv vs autograd {c}")


def pin_backward_chunks_sum_to_full(orc):
    """Per-chunk-pair contributions with the full-row lse sum to the full gradients."""
    for P, n, B, Hq, Hkv, d, causal, scale, seed in [(3, 4, 1, 2, 1, 3, True, 0.9, 51), (2, 5, 1, 4, 2, 2, False, 1.2, 52),
                                                     (4, 2, 2, 2, 2, 2, True, 1.0, 53)]:
        rng = np.random.default_rng(seed)
        L = P * n
        q = rng.standard_normal((B, Hq, L, d))
        k = rng.standard_normal((B, Hkv, L, d)) * 1.5
        v = rng.standard_normal((B, Hkv, L, d))
        do = rng.standard_normal((B, Hq, L, d))
        dq, dk, dv = orc.attention_bwd_fp64(q, k, v, do, scale=scale, causal=causal)
        O, lse = orc.attention_fp64(q, k, v, scale=scale, causal=causal)
        D = orc.rowsum_do_o_fp64(do, O)
        cq, ck, cv = np.zeros_like(dq), np.zeros_like(dk), np.zeros_like(dv)
        for i in range(P):
            qs = slice(i * n, (i + 1) * n)
            for j in range(P):
                ks = slice(j * n, (j + 1) * n)
                a, b_, c_ = orc.chunk_attention_bwd_fp64(q[:, :, qs], k[:, :, ks], v[:, :, ks], do[:, :, qs],
                                                          lse[:, :, qs], D[:, :, qs], scale=scale, causal=causal,
                                                          q_pos0=i * n, k_pos0=j * n)
                cq[:, :, qs] += a
                ck[:, :, ks] += b_
                cv[:, :, ks] += c_
        _close(cq, dq, 1e-12, f"chunked dq P={P}")
        _close(ck, dk, 1e-12, f"chunked dk P={P}")
        _close(cv, dv, 1e-12, f"chunked dv P={P}")
        # D is rowsum(P * dP) as well (a property of the softmax Jacobian)
        Ddirect = np.zeros_like(D)
        grp = Hq // Hkv
        for b in range(B):
            for h in range(Hq):
                g = h // grp
                s = scale * (q[b, h] @ k[b, g].T)
                if causal:
                    s = np.where(np.arange(L)[None, :] <= np.arange(L)[:, None], s, -np.inf)
                p = np.exp(s - lse[b, h][:, None])
                Ddirect[b, h] = (p * (do[b, h] @ v[b, g].T)).sum(axis=1)
        _close(D, Ddirect, 1e-12, "D = rowsum(P * dP)")


# ----------------------------------------------------------------------------
# packed samples
# ----------------------------------------------------------------------------
def pin_packed_equals_separate_samples(orc):
    """Attention over a packed sequence equals causal attention run on every
    sample by itself (the samples never see each other)."""
    rng = np.random.default_rng(61)
    for L, starts, Hq, Hkv, d in [(12, [0, 5, 6, 9], 2, 1, 3), (10, [0], 2, 2, 2), (9, [0, 1, 2, 3, 4, 5, 6, 7, 8], 1, 1, 2),
                                  (16, [0, 8], 4, 2, 3)]:
        q = rng.standard_normal((1, Hq, L, d))
        k = rng.standard_normal((1, Hkv, L, d)) * 1.5
        v = rng.standard_normal((1, Hkv, L, d))
        O, lse = orc.attention_packed_fp64(q, k, v, starts, scale=0.9)
        ends = list(starts[1:]) + [L]
        for s0, s1 in zip(starts, ends):
            Os, ls = orc.attention_fp64(q[:, :, s0:s1], k[:, :, s0:s1], v[:, :, s0:s1], scale=0.9, causal=True)
            _close(O[:, :, s0:s1], Os, 1e-12, f"packed O sample {s0}..{s1}")
            _close(lse[:, :, s0:s1], ls, 1e-12, f"packed lse sample {s0}..{s1}")
        ids = orc.segment_ids(L, starts)
        assert ids.tolist() == [sum(1 for s in starts if s <= t) - 1 for t in range(L)]
    for bad in ([1, 3], [0, 3, 3], [0, 12]):
        try:
            orc.segment_ids(12, bad)
        except ValueError:
            pass
        else:
            raise AssertionError(f"bad sample starts {bad} accepted")


def pin_closed_form(orc):
    g = _load("attn_matrix_memory.json")
    b = orc.attn_matrix_bytes(g["L"], g["heads"], g["elem_bytes"])
    assert b == g["exact_bytes_per_head"]
    assert abs(b / 2**30 - g["printed_GB_per_head"]) < 0.5
    assert orc.attn_matrix_bytes(1024, 32, 2) == 1024 * 1024 * 2 * 32


ALL_PINS = [
    pin_attention_bruteforce,
    pin_attention_sdpa,
    pin_attention_closed_forms,
    pin_attention_hand_golden,
    pin_unmasked_pairs,
    pin_merge_algebra,
    pin_ring_equals_full,
    pin_ring_visit_order,
    pin_ulysses_hand_golden,
    pin_ulysses_library_form,
    pin_ulysses_roundtrip_tags,
    pin_ulysses_replication,
    pin_ulysses_limits,
    pin_closed_form,
    pin_attention_at_positions,
    pin_zigzag_positions,
    pin_zigzag_equals_full,
    pin_zigzag_balance,
    pin_backward_finite_differences,
    pin_backward_autograd,
    pin_backward_chunks_sum_to_full,
    pin_packed_equals_separate_samples,
]

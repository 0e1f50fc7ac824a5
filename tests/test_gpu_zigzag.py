"""Zigzag causal ring attention (ra_zigzag_attention) against the fp64 oracle.

Every rank's shard of a small sequence is compared element by element with the
oracle's causal attention at the zigzag positions; shapes cover P = 1 (the
whole sequence on one rank), odd P, ragged pieces that end inside a 64-key
tile, GQA, both head dims, bf16 and fp32 inputs.  The full-size 128k ring is
checked on sampled rows of the first and last rank."""
import numpy as np
import pytest

import oracle
from sequence_kv_chunk_amd.synth import WORKLOADS, attention_inputs, bf16_bits_to_f64, f32_to_bf16_bits

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from gpu_util import check_close, dev_bf16, dev_f32, host_f64, say  # noqa: E402


@pytest.fixture(scope="module")
def api():
    from sequence_kv_chunk_amd import api
    return api


CASES = [
    # P, c (piece length), B, Hq, Hkv, d, dtype, out dtype
    (1, 64, 1, 2, 2, 128, "bf16", "bf16"),
    (2, 100, 1, 4, 2, 128, "bf16", "f32"),
    (3, 257, 1, 2, 1, 128, "bf16", "bf16"),
    (4, 64, 2, 4, 4, 64, "bf16", "bf16"),
    (8, 48, 1, 2, 2, 128, "bf16", "bf16"),
    (4, 40, 1, 4, 2, 64, "f32", "f32"),
    # 256 query heads: the fp32 launches take the shared-tile kernel (the
    # third launch walks the pool backwards, with a negative chunk stride)
    (4, 130, 1, 256, 32, 128, "f32", "f32"),
    (3, 64, 1, 256, 64, 64, "f32", "f32"),
]


@pytest.mark.parametrize("case", CASES, ids=[f"P{c[0]}_c{c[1]}_d{c[5]}_{c[6]}" for c in CASES])
def test_zigzag_small(api, case):
    P, c, B, Hq, Hkv, d, dt, odt = case
    say(f"zigzag {case}")
    n = 2 * c
    rng = np.random.default_rng(1000 + P * 31 + c)
    q = rng.standard_normal((P, B, Hq, n, d), dtype=np.float32) * np.float32(d ** -0.5)
    k = rng.standard_normal((P, B, Hkv, n, d), dtype=np.float32)
    v = rng.standard_normal((P, B, Hkv, n, d), dtype=np.float32)
    if dt == "bf16":
        qb, kb, vb = (f32_to_bf16_bits(x) for x in (q, k, v))
        qh, kh, vh = (bf16_bits_to_f64(x) for x in (qb, kb, vb))
        qd, kd, vd = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb)
    else:
        qh, kh, vh = (x.astype(np.float64) for x in (q, k, v))
        qd, kd, vd = dev_f32(q), dev_f32(k), dev_f32(v)
    tdt = torch.bfloat16 if odt == "bf16" else torch.float32
    for r in range(P):
        o = torch.full((B, Hq, n, d), float("nan"), dtype=tdt, device="cuda")
        lse = torch.full((B * Hq * n,), float("nan"), dtype=torch.float32, device="cuda")
        work = (torch.full((B, Hq, c, d), float("nan"), dtype=torch.float32, device="cuda"),
                torch.full((B * Hq * c,), float("nan"), dtype=torch.float32, device="cuda"))
        api.ra_zigzag_attention(qd[r], kd, vd, o, lse, rank=r, work=work)
        torch.cuda.synchronize()
        ref_o, ref_l = oracle.zigzag_attention_fp64(qh[r], kh, vh, r)
        tol = "f32" if dt == "f32" else "bf16"
        check_close(host_f64(o), ref_o, tol, f"O rank {r}")
        check_close(host_f64(lse).reshape(B, Hq, n), ref_l, tol, f"lse rank {r}")


@pytest.mark.slow
def test_zigzag_128k_full(api):
    """All 8 ranks of the causal 128k zigzag ring; rows sampled on ranks 0 and 7."""
    w = WORKLOADS["zigzag_bf16_128k_causal"]
    say(f"full size {w.name}")
    x = attention_inputs(w)
    kd, vd = dev_bf16(x["k"]), dev_bf16(x["v"])
    rng = np.random.default_rng(66)
    heads = [0, w.Hq - 1, int(rng.integers(1, w.Hq - 1))]
    n, c = w.n, w.n // 2
    kh = bf16_bits_to_f64(x["k"][:, :, heads])
    vh = bf16_bits_to_f64(x["v"][:, :, heads])
    for r in (0, w.P - 1):
        qd = dev_bf16(x["q"][r])
        o = torch.full((w.B, w.Hq, n, w.d), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty(w.B * w.Hq * n, dtype=torch.float32, device="cuda")
        api.ra_zigzag_attention(qd, kd, vd, o, lse, rank=r)
        torch.cuda.synchronize()
        oh = host_f64(o)[:, heads]
        lh = host_f64(lse).reshape(w.B, w.Hq, n)[:, heads]
        rows = sorted({0, c - 1, c, n - 1} | {int(t) for t in rng.integers(0, n, size=6)})
        kp = np.concatenate([oracle.zigzag_positions(j, w.P, c) for j in range(w.P)])
        kall = np.concatenate([kh[j] for j in range(w.P)], axis=2)
        vall = np.concatenate([vh[j] for j in range(w.P)], axis=2)
        qpos = oracle.zigzag_positions(r, w.P, c)
        for t in rows:
            qh = bf16_bits_to_f64(x["q"][r][:, heads][:, :, t:t + 1])
            ref_o, ref_l = oracle.attention_at_positions_fp64(qh, kall, vall, qpos[t:t + 1], kp)
            check_close(oh[:, :, t:t + 1], ref_o, "bf16", f"O rank {r} row {t}")
            check_close(lh[:, :, t:t + 1], ref_l, "bf16", f"lse rank {r} row {t}")

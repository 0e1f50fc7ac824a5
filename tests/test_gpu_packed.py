"""Causal ring attention over packed samples (ra_ring_attention_packed)
against the fp64 oracle: every rank of small rings, with samples that span
chunk boundaries, start exactly on chunk and tile boundaries, are one token
long or cover the whole sequence."""
import numpy as np
import pytest

import oracle
from sequence_kv_chunk_amd.synth import bf16_bits_to_f64, f32_to_bf16_bits

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from gpu_util import check_close, dev_bf16, host_f64, say  # noqa: E402


@pytest.fixture(scope="module")
def api():
    from sequence_kv_chunk_amd import api
    return api


CASES = [
    # P, n, Hq, Hkv, d, sample starts
    (4, 256, 2, 2, 128, [0]),                                       # one sample: the plain causal ring
    (4, 256, 4, 2, 128, [0, 100, 400, 401, 700, 1000]),             # samples across chunk boundaries
    (4, 256, 2, 1, 128, [0, 256, 512, 768]),                        # one sample per chunk
    (2, 300, 2, 2, 64, list(range(0, 600, 17))),                    # many short samples, ragged chunks
    (1, 700, 2, 2, 128, [0, 64, 128, 129, 511, 512, 699]),          # one chunk; tile-aligned starts
    (8, 128, 2, 2, 128, [0, 5, 900]),                               # a sample over seven chunks
    (3, 200, 4, 2, 64, [0, 70, 333, 450], 2),                       # two batch rows, one packing
]


@pytest.mark.parametrize("case", CASES, ids=[f"P{c[0]}_n{c[1]}_s{len(c[5])}" + (f"_B{c[6]}" if len(c) > 6 else "")
                                             for c in CASES])
def test_packed_ring(api, case):
    P, n, Hq, Hkv, d, starts = case[:6]
    B = case[6] if len(case) > 6 else 1
    say(f"packed {case[:5]} B={B} {len(starts)} samples")
    L = P * n
    rng = np.random.default_rng(5000 + L + len(starts))
    qb = f32_to_bf16_bits(rng.standard_normal((P, B, Hq, n, d), dtype=np.float32) * np.float32(d ** -0.5))
    kb = f32_to_bf16_bits(rng.standard_normal((P, B, Hkv, n, d), dtype=np.float32))
    vb = f32_to_bf16_bits(rng.standard_normal((P, B, Hkv, n, d), dtype=np.float32))
    full = lambda x: bf16_bits_to_f64(x).transpose(1, 2, 0, 3, 4).reshape(B, x.shape[2], L, d)
    ref_o, ref_l = oracle.attention_packed_fp64(full(qb), full(kb), full(vb), starts)
    kd, vd = dev_bf16(kb), dev_bf16(vb)
    seg = torch.tensor(starts, dtype=torch.int64, device="cuda")
    for r in range(P):
        o = torch.full((B, Hq, n, d), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full((B * Hq * n,), float("nan"), dtype=torch.float32, device="cuda")
        api.ra_ring_attention_packed(dev_bf16(qb[r]), kd, vd, o, lse, seg, rank=r)
        torch.cuda.synchronize()
        check_close(host_f64(o), ref_o[:, :, r * n:(r + 1) * n], "bf16", f"O rank {r}")
        check_close(host_f64(lse).reshape(B, Hq, n), ref_l[:, :, r * n:(r + 1) * n], "bf16", f"lse rank {r}")


def test_packed_fast_pass_fallback(api):
    """Scores near +384 (weights past float's range without a shift) on one head:
    its workgroups redo the visit with the running maximum; the other head's
    do not."""
    P, n, H, d, starts = 2, 300, 2, 128, [0, 150, 451]
    say("packed fast-pass fallback")
    L = P * n
    rng = np.random.default_rng(77)
    q = rng.standard_normal((P, 1, H, n, d), dtype=np.float32) * np.float32(d ** -0.5)
    k = rng.standard_normal((P, 1, H, n, d), dtype=np.float32)
    u = rng.standard_normal(d, dtype=np.float32)        # head 0: every score near +384 (nats)
    q[:, :, 0] = np.float32(3.0) * u + np.float32(0.3 * d ** 0.5) * q[:, :, 0]
    k[:, :, 0] = u + np.float32(0.3) * k[:, :, 0]
    qb = f32_to_bf16_bits(q)
    kb = f32_to_bf16_bits(k)
    vb = f32_to_bf16_bits(rng.standard_normal((P, 1, H, n, d), dtype=np.float32))
    full = lambda x: bf16_bits_to_f64(x).transpose(1, 2, 0, 3, 4).reshape(1, x.shape[2], L, d)
    ref_o, ref_l = oracle.attention_packed_fp64(full(qb), full(kb), full(vb), starts)
    kd, vd = dev_bf16(kb), dev_bf16(vb)
    seg = torch.tensor(starts, dtype=torch.int64, device="cuda")
    for r in range(P):
        o = torch.full((1, H, n, d), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full((H * n,), float("nan"), dtype=torch.float32, device="cuda")
        api.ra_ring_attention_packed(dev_bf16(qb[r]), kd, vd, o, lse, seg, rank=r)
        torch.cuda.synchronize()
        check_close(host_f64(o), ref_o[:, :, r * n:(r + 1) * n], "bf16", f"O rank {r}")
        check_close(host_f64(lse).reshape(1, H, n), ref_l[:, :, r * n:(r + 1) * n], "bf16", f"lse rank {r}")


@pytest.mark.parametrize("Hq,Hkv,d,starts", [
    (1024, 128, 128, [0, 37, 250, 251, 333, 512, 600, 639]),
    (512, 512, 64, [0, 31, 64, 256, 257, 300, 320, 321, 480]),
], ids=["h1024_d128", "h512_d64"])
def test_packed_many_visits_per_workgroup(api, Hq, Hkv, d, starts):
    """Enough heads that every workgroup makes several visits in turn (each
    visit loads the next one's first tiles before its own stores): every
    output finite, and sampled heads against the oracle in full."""
    P, n = 2, 320
    L = P * n
    say(f"packed, {Hq} heads, d={d}: several visits per workgroup")
    rng = np.random.default_rng(5100 + Hq + d)
    qb = f32_to_bf16_bits(rng.standard_normal((P, 1, Hq, n, d), dtype=np.float32) * np.float32(d ** -0.5))
    kb = f32_to_bf16_bits(rng.standard_normal((P, 1, Hkv, n, d), dtype=np.float32))
    vb = f32_to_bf16_bits(rng.standard_normal((P, 1, Hkv, n, d), dtype=np.float32))
    heads = np.unique(np.concatenate([[0, 1, Hq - 1], rng.integers(0, Hq, size=45)]))
    kv = heads // (Hq // Hkv)
    full = lambda x, sel: bf16_bits_to_f64(x[:, :, sel]).transpose(1, 2, 0, 3, 4).reshape(1, len(sel), L, d)
    ref_o, ref_l = oracle.attention_packed_fp64(full(qb, heads), full(kb, kv), full(vb, kv), starts)
    kd, vd = dev_bf16(kb), dev_bf16(vb)
    seg = torch.tensor(starts, dtype=torch.int64, device="cuda")
    for r in range(P):
        o = torch.full((1, Hq, n, d), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full((Hq * n,), float("nan"), dtype=torch.float32, device="cuda")
        api.ra_ring_attention_packed(dev_bf16(qb[r]), kd, vd, o, lse, seg, rank=r)
        torch.cuda.synchronize()
        go, gl = host_f64(o), host_f64(lse).reshape(1, Hq, n)
        assert np.isfinite(go).all() and np.isfinite(gl).all(), f"rank {r}: unwritten or non-finite outputs"
        check_close(go[:, heads], ref_o[:, :, r * n:(r + 1) * n], "bf16", f"O rank {r}")
        check_close(gl[:, heads], ref_l[:, :, r * n:(r + 1) * n], "bf16", f"lse rank {r}")


@pytest.mark.slow
def test_packed_32k_full_sampled(api):
    """The 32k ring packing 16 samples of 2048 tokens, the shape bench.py
    times (8 ranks x 4096 tokens, 32 heads, d = 128): sampled rows of every
    rank against the oracle's softmax over the row's own sample prefix."""
    from sequence_kv_chunk_amd.synth import WORKLOADS, attention_inputs
    w = WORKLOADS["ring_bf16_32k"]
    say(f"packed full size {w.name}, samples of 2048")
    x = attention_inputs(w)
    P, n, H, d, L = w.P, w.n, w.Hq, w.d, w.L
    seg_len = 2048
    seg = torch.arange(0, L, seg_len, dtype=torch.int64, device="cuda")
    kd, vd = dev_bf16(x["k"]), dev_bf16(x["v"])
    kf = x["k"].transpose(1, 2, 0, 3, 4).reshape(H, L, d)          # [H, L, d] bits, natural order
    vf = x["v"].transpose(1, 2, 0, 3, 4).reshape(H, L, d)
    rng = np.random.default_rng(6000)
    for r in range(P):
        o = torch.full((1, H, n, d), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full((H * n,), float("nan"), dtype=torch.float32, device="cuda")
        api.ra_ring_attention_packed(dev_bf16(x["q"][r]), kd, vd, o, lse, seg, rank=r)
        torch.cuda.synchronize()
        go, gl = host_f64(o)[0], host_f64(lse).reshape(H, n)
        rows = sorted({0, 1, seg_len - 1, seg_len, n - 1, *(int(i) for i in rng.integers(0, n, size=2))})
        for h in (0, 17, H - 1):
            for row in rows:
                t = r * n + row
                s0 = (t // seg_len) * seg_len
                qr = bf16_bits_to_f64(x["q"][r][0, h, row])[None, None, None]
                ref_o, ref_l = oracle.attention_fp64(qr, bf16_bits_to_f64(kf[h, s0:t + 1])[None, None],
                                                     bf16_bits_to_f64(vf[h, s0:t + 1])[None, None])
                check_close(go[h, row][None, None, None], ref_o, "bf16", f"O rank {r} row {row} head {h}")
                check_close(np.array([[[gl[h, row]]]]), ref_l, "bf16", f"lse rank {r} row {row} head {h}")

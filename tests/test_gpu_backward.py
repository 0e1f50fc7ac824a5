"""Attention backward (bf16 MFMA kernels) against the fp64 oracle.

One chunk pair at a time with the oracle's lse and D as inputs (so that the
kernels are checked on their own), the D preprocess, and the whole ring
backward end to end (GPU forward, GPU D, every rank's backward accumulated)
against the gradients of full attention.  Tolerance for the fp32 gradients
of bf16 inputs: max-abs error <= 2e-2 * max(1, max |reference|) per tensor
(the attention bar, scaled to the gradient's magnitude)."""
import numpy as np
import pytest

import oracle
from sequence_kv_chunk_amd.synth import bf16_bits_to_f64, f32_to_bf16_bits

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from gpu_util import dev_bf16, host_f64, say  # noqa: E402

GRAD_TOL = 2e-2


def check_grad(got, ref, what):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, f"{what}: shape {got.shape} vs {ref.shape}"
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    err = float(np.max(np.abs(got - ref))) if got.size else 0.0
    bound = GRAD_TOL * max(1.0, float(np.max(np.abs(ref))) if ref.size else 1.0)
    assert err <= bound, f"{what}: max abs err {err:.3e} > {bound:.3e}"
    say(f"   {what}: max abs err {err:.2e} (max |ref| {float(np.max(np.abs(ref))):.2e})")
    return err


@pytest.fixture(scope="module")
def api():
    from sequence_kv_chunk_amd import api
    return api


def _bits(shape, rng, scale=1.0):
    return f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32) * np.float32(scale))


CASES = [
    # B, Hq, Hkv, nq, nk, d, causal, q_pos0, k_pos0, scale
    (1, 2, 2, 64, 64, 128, False, 0, 0, 1.0),
    (1, 2, 1, 100, 70, 128, False, 0, 0, 1.0),
    (2, 4, 2, 300, 200, 64, False, 0, 0, 0.8),
    (1, 2, 2, 257, 257, 128, True, 0, 0, 1.0),       # diagonal block, ragged
    (1, 4, 1, 200, 300, 128, True, 500, 300, 1.0),   # queries ahead of the keys
    (1, 2, 2, 130, 200, 64, True, 0, 60, 1.0),       # first rows see nothing
    (1, 8, 2, 129, 513, 128, False, 0, 0, 1.2),      # GQA 4:1, several key tiles
    (1, 2, 2, 1, 1, 128, False, 0, 0, 1.0),          # one query, one key
    (1, 4, 2, 3, 200, 64, False, 0, 0, 0.7),         # three queries, ragged keys
    (1, 2, 1, 70, 40, 128, True, 0, 100, 1.0),       # every key after every query: no contribution
    (2, 2, 2, 200, 1, 128, True, 50, 0, 1.0),        # one key, seen by every row
    (1, 2, 2, 600, 600, 64, True, 0, 0, 1.0),        # diagonal over several query and key workgroups
    (1, 4, 2, 700, 450, 128, True, 0, 200, 1.0),     # key workgroups whose walks start at different tiles
    (2, 4, 1, 520, 260, 128, False, 0, 0, 0.9),      # GQA 4:1, B=2, ragged query and key tails
    (2, 8, 1, 300, 520, 64, True, 100, 0, 1.1),      # GQA 8:1 at d=64, B=2, queries ahead of the keys
    (1, 3, 3, 64, 1000, 128, False, 0, 0, 1.0),      # one query tile, eight key workgroups, odd head count
]


@pytest.mark.parametrize("case", CASES, ids=[f"c{i}" for i in range(len(CASES))])
def test_chunk_bwd(api, case):
    B, Hq, Hkv, nq, nk, d, causal, qp, kp, scale = case
    say(f"chunk bwd {case}")
    rng = np.random.default_rng(700 + nq + nk + d)
    qb = _bits((B, Hq, nq, d), rng, d ** -0.5)
    kb = _bits((B, Hkv, nk, d), rng)
    vb = _bits((B, Hkv, nk, d), rng)
    ob = _bits((B, Hq, nq, d), rng)
    q, k, v, do = (bf16_bits_to_f64(x) for x in (qb, kb, vb, ob))
    # the rows' lse and D as a full forward over these keys would give them
    O, lse = oracle.attention_fp64(q, k, v, scale=scale, causal=causal, q_pos0=qp, k_pos0=kp)
    D = oracle.rowsum_do_o_fp64(do, O)
    ref = oracle.chunk_attention_bwd_fp64(q, k, v, do, lse, D, scale=scale, causal=causal, q_pos0=qp, k_pos0=kp)
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()
    dq = torch.zeros((B, Hq, nq, d), dtype=torch.float32, device="cuda")
    dk = torch.zeros((B, Hkv, nk, d), dtype=torch.float32, device="cuda")
    dv = torch.zeros_like(dk)
    api.ra_chunk_attention_bwd(dev_bf16(qb), dev_bf16(kb), dev_bf16(vb), dev_bf16(ob), dev(lse).reshape(-1),
                               dev(D).reshape(-1), dq, dk, dv, scale=scale, causal=causal, q_pos0=qp, k_pos0=kp)
    torch.cuda.synchronize()
    for name, g, r in (("dq", dq, ref[0]), ("dk", dk, ref[1]), ("dv", dv, ref[2])):
        check_grad(host_f64(g), r, f"{name} {case}")


def test_bwd_preprocess(api):
    rng = np.random.default_rng(77)
    for dt in ("bf16", "f32"):
        for d in (64, 128):
            x = rng.standard_normal((2, 3, 70, d), dtype=np.float32)
            y = rng.standard_normal((2, 3, 70, d), dtype=np.float32)
            if dt == "bf16":
                xb, yb = f32_to_bf16_bits(x), f32_to_bf16_bits(y)
                xd, yd = dev_bf16(xb), dev_bf16(yb)
                ref = oracle.rowsum_do_o_fp64(bf16_bits_to_f64(yb), bf16_bits_to_f64(xb))
            else:
                xd, yd = torch.from_numpy(x).cuda(), torch.from_numpy(y).cuda()
                ref = oracle.rowsum_do_o_fp64(y, x)
            D = torch.full((2 * 3 * 70,), float("nan"), dtype=torch.float32, device="cuda")
            api.ra_attention_bwd_preprocess(xd, yd, D)
            torch.cuda.synchronize()
            got = host_f64(D).reshape(2, 3, 70)
            assert np.max(np.abs(got - ref)) <= 1e-5 * max(1.0, np.max(np.abs(ref))), (dt, d)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("P,n,Hq,Hkv,d", [(4, 128, 4, 2, 128), (3, 100, 2, 2, 64), (1, 200, 2, 1, 128),
                                          (3, 300, 2, 1, 128)])
def test_ring_bwd_end_to_end(api, P, n, Hq, Hkv, d, causal):
    """GPU ring forward, GPU D, every rank's GPU backward; against the
    gradients of one softmax over the whole sequence."""
    say(f"ring bwd P={P} n={n} causal={causal}")
    B = 1
    rng = np.random.default_rng(900 + P * n + d + int(causal))
    qb = _bits((P, B, Hq, n, d), rng, d ** -0.5)
    kb = _bits((P, B, Hkv, n, d), rng)
    vb = _bits((P, B, Hkv, n, d), rng)
    ob = _bits((P, B, Hq, n, d), rng)
    _ring_bwd_check(api, qb, kb, vb, ob, causal)


@pytest.mark.parametrize("causal", [False, True])
def test_rounding_edge_ring_bwd(api, causal):
    """The ring backward fed by the GPU forward's lse on inputs whose scores
    all sit at 9-17 nats, aligned with their queries (row sums 2^20-2^36, the
    range where the forward keeps its fast pass): P = exp(S - lse) scales
    every gradient by any error in lse."""
    from sequence_kv_chunk_amd.synth import aligned_score_inputs
    P, B, H, n, d = 4, 1, 2, 256, 128
    say(f"ring bwd, rounding edge inputs, causal={causal}")
    qb, kb, vb = aligned_score_inputs(B, H, P * n, P * n, d, seed=80 + int(causal))
    pool = lambda x: np.ascontiguousarray(x.reshape(B, H, P, n, d).transpose(2, 0, 1, 3, 4))
    ob = _bits((P, B, H, n, d), np.random.default_rng(81))
    _ring_bwd_check(api, pool(qb), pool(kb), pool(vb), ob, causal)


def _ring_bwd_check(api, qb, kb, vb, ob, causal):
    """GPU ring forward, D and backward of every rank of pools [P, B, H, n, d]
    against the gradients of one softmax over the whole sequence."""
    P, B, Hq, n, d = qb.shape
    Hkv = kb.shape[2]
    full = lambda x: bf16_bits_to_f64(x).transpose(1, 2, 0, 3, 4).reshape(B, x.shape[2], P * n, d)
    ref = oracle.attention_bwd_fp64(full(qb), full(kb), full(vb), full(ob), causal=causal)
    kd, vd = dev_bf16(kb), dev_bf16(vb)
    dk = torch.zeros((P, B, Hkv, n, d), dtype=torch.float32, device="cuda")
    dv = torch.zeros_like(dk)
    for r in range(P):
        qd, od = dev_bf16(qb[r]), dev_bf16(ob[r])
        o = torch.empty((B, Hq, n, d), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty(B * Hq * n, dtype=torch.float32, device="cuda")
        api.ra_ring_attention(qd, kd, vd, o, lse, rank=r, causal=causal)
        D = torch.empty_like(lse)
        api.ra_attention_bwd_preprocess(o, od, D)
        dq = torch.zeros((B, Hq, n, d), dtype=torch.float32, device="cuda")
        api.ra_ring_attention_bwd(qd, kd, vd, od, lse, D, dq, dk, dv, rank=r, causal=causal)
        torch.cuda.synchronize()
        check_grad(host_f64(dq), ref[0][:, :, r * n:(r + 1) * n], f"dq rank {r}")
    dkf = host_f64(dk).transpose(1, 2, 0, 3, 4).reshape(B, Hkv, P * n, d)
    dvf = host_f64(dv).transpose(1, 2, 0, 3, 4).reshape(B, Hkv, P * n, d)
    check_grad(dkf, ref[1], "dk pool")
    check_grad(dvf, ref[2], "dv pool")


@pytest.mark.slow
def test_ring_bwd_32k_full_sampled(api):
    """The backward of the whole 32k ring (8 ranks x 8 resident chunks of
    4096, 32 heads, d=128, the shape and launch sequence bench.py times),
    checked on sampled query rows (dQ) and sampled keys (dK, dV) of two heads.
    The oracle works from its own full-row lse and D (one softmax per row over
    all 32768 keys), so none of its inputs comes from the GPU."""
    from sequence_kv_chunk_amd.synth import WORKLOADS, attention_inputs
    w = WORKLOADS["ring_bf16_32k"]
    say(f"full-size backward {w.name}")
    x = attention_inputs(w)
    P, n, d, H, B = w.P, w.n, w.d, w.Hq, w.B
    rng = np.random.default_rng(777)
    ob = _bits(x["q"].shape, rng)
    kd, vd = dev_bf16(x["k"]), dev_bf16(x["v"])
    dk = torch.zeros(x["k"].shape, dtype=torch.float32, device="cuda")
    dv = torch.zeros_like(dk)
    dqs = []
    for r in range(P):
        qd, od = dev_bf16(x["q"][r]), dev_bf16(ob[r])
        o = torch.empty((B, H, n, d), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty(B * H * n, dtype=torch.float32, device="cuda")
        api.ra_ring_attention(qd, kd, vd, o, lse, rank=r, causal=False)
        D = torch.empty_like(lse)
        api.ra_attention_bwd_preprocess(o, od, D)
        dq = torch.zeros((B, H, n, d), dtype=torch.float32, device="cuda")
        api.ra_ring_attention_bwd(qd, kd, vd, od, lse, D, dq, dk, dv, rank=r, causal=False)
        dqs.append(dq)
    torch.cuda.synchronize()

    heads = [0, H - 1]
    full = lambda bits: bf16_bits_to_f64(bits[:, :, heads]).transpose(1, 2, 0, 3, 4).reshape(B, len(heads), P * n, d)
    qf, kf, vf, of = full(x["q"]), full(x["k"]), full(x["v"]), full(ob)
    o_ref, lse_ref = oracle.attention_fp64(qf, kf, vf)
    D_ref = oracle.rowsum_do_o_fp64(of, o_ref)
    pick = lambda: sorted({0, 1, n - 1, n, P * n - 1, *(int(i) for i in rng.integers(0, P * n, size=8))})
    rows, keys = pick(), pick()

    dq_ref, _, _ = oracle.chunk_attention_bwd_fp64(qf[:, :, rows], kf, vf, of[:, :, rows],
                                                   lse_ref[:, :, rows], D_ref[:, :, rows])
    dq_got = np.stack([host_f64(dqs[r // n][:, heads][:, :, r % n]) for r in rows], axis=2)
    check_grad(dq_got, dq_ref, "dq sampled rows")

    _, dk_ref, dv_ref = oracle.chunk_attention_bwd_fp64(qf, kf[:, :, keys], vf[:, :, keys], of, lse_ref, D_ref)
    dk_got = np.stack([host_f64(dk[j // n][:, heads][:, :, j % n]) for j in keys], axis=2)
    dv_got = np.stack([host_f64(dv[j // n][:, heads][:, :, j % n]) for j in keys], axis=2)
    check_grad(dk_got, dk_ref, "dk sampled keys")
    check_grad(dv_got, dv_ref, "dv sampled keys")

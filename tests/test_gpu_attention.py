"""Chunked attention kernels (fp32 and bf16 MFMA) against the fp64 oracle.

Small cases are compared element by element over whole outputs; shapes span
several 256-row query tiles and 64-key tiles with ragged tails, causal
diagonals at different offsets, fully masked rows, GQA ratios and both head
dims.  The full-size workloads (32k ring, rank 7 of a causal 128k ring, one
128k Ulysses share) are checked whole for finiteness and, in every head, on
the first and last row of every 256-row query tile plus random rows, which
the oracle computes against all the keys each row sees."""
import math

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


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape, dtype=np.float32) * np.float32(scale)


def _inputs(dtype, B, Hq, Hkv, nq, nk, d, seed, qscale=None, kramp=False):
    """Q, K, V as host float64 (exact values) plus device tensors."""
    qs = (1.0 / math.sqrt(d)) if qscale is None else qscale
    q = _rand((B, Hq, nq, d), seed, qs)
    k = _rand((B, Hkv, nk, d), seed + 1)
    v = _rand((B, Hkv, nk, d), seed + 2)
    if kramp:  # keys grow along the sequence: the running max keeps rising
        k *= (0.05 + np.arange(nk, dtype=np.float32) / 400.0)[None, None, :, None]
    if dtype == "bf16":
        bits = [f32_to_bf16_bits(x) for x in (q, k, v)]
        host = [bf16_bits_to_f64(b) for b in bits]
        dev = [dev_bf16(b) for b in bits]
    else:
        host = [x.astype(np.float64) for x in (q, k, v)]
        dev = [dev_f32(x) for x in (q, k, v)]
    return host, dev


def _out(B, H, n, d, dtype):
    o = torch.full((B, H, n, d), float("nan"), dtype=dtype, device="cuda")
    lse = torch.full((B * H * n,), float("nan"), dtype=torch.float32, device="cuda")
    return o, lse


CHUNK_CASES = [
    # B, Hq, Hkv, nq, nk, d, causal, q_pos0, k_pos0, scale
    (1, 2, 2, 1, 1, 64, False, 0, 0, 1.0),
    (1, 2, 2, 100, 65, 128, False, 0, 0, 1.0),
    (2, 4, 2, 300, 200, 64, False, 0, 0, 0.7),
    (1, 8, 1, 257, 1000, 128, False, 0, 0, 1.0),
    (1, 4, 4, 513, 513, 128, True, 0, 0, 1.0),      # diagonal block, ragged
    (1, 4, 2, 256, 256, 64, True, 0, 0, 1.3),
    (1, 2, 2, 300, 700, 128, True, 500, 0, 1.0),    # queries ahead of the keys
    (1, 2, 1, 200, 300, 128, True, 0, 100, 1.0),    # first 100 rows see nothing
    (1, 2, 2, 64, 64, 128, True, 0, 1000, 1.0),     # every row masked
    (2, 16, 2, 130, 129, 128, True, 129, 0, 0.9),   # GQA 8:1
    (1, 4, 1, 1024, 1024, 128, False, 0, 0, 1.0),   # several full tiles
]


def _ids(cases):
    return ["B{}Hq{}Hkv{}nq{}nk{}d{}{}q{}k{}".format(*c[:6], "c" if c[6] else "n", c[7], c[8]) for c in cases]


@pytest.mark.parametrize("in_dt", ["f32", "bf16"])
@pytest.mark.parametrize("case", CHUNK_CASES, ids=_ids(CHUNK_CASES))
def test_chunk_partial(api, case, in_dt):
    B, Hq, Hkv, nq, nk, d, causal, qp, kp, scale = case
    say(f"chunk partial {in_dt} {case}")
    (q, k, v), (qd, kd, vd) = _inputs(in_dt, B, Hq, Hkv, nq, nk, d, seed=nq + nk + d)
    ref_o, ref_l = oracle.attention_fp64(q, k, v, scale=scale, causal=causal, q_pos0=qp, k_pos0=kp)
    out_dts = [torch.float32] if in_dt == "f32" else [torch.float32, torch.bfloat16]
    for odt in out_dts:
        o, lse = _out(B, Hq, nq, d, odt)
        api.ra_chunk_attention(qd, kd, vd, o, lse, scale=scale, causal=causal, q_pos0=qp, k_pos0=kp)
        torch.cuda.synchronize()
        tol = "bf16" if (in_dt == "bf16" or odt == torch.bfloat16) else "f32"
        check_close(host_f64(o), ref_o, tol, f"O ({odt})")
        check_close(host_f64(lse).reshape(ref_l.shape), ref_l, tol, "lse")


@pytest.mark.parametrize("Hq", [4, 256], ids=["split_kernel", "shared_kernel"])
@pytest.mark.parametrize("d", [64, 128])
def test_f32_overlapping_key_rows(api, d, Hq):
    """fp32 keys and values whose rows overlap in memory (row stride d/2: a
    window sliding over one buffer, and a single row repeated with stride 0
    for the values): every tile copy must read each row's whole d values,
    not row count x row stride bytes.  4 query heads take the small-launch
    fp32 kernel, 256 the shared-tile one."""
    B, Hkv, nq, nk = 1, 2, 150, 77
    say(f"f32 overlapping key/value rows, d={d}, Hq={Hq}")
    rng = np.random.default_rng(6100 + d)
    q = rng.standard_normal((B, Hq, nq, d), dtype=np.float32) * np.float32(d ** -0.5)
    flat_k = rng.standard_normal(Hkv * (nk * d // 2 + d), dtype=np.float32)
    flat_v = rng.standard_normal(Hkv * d, dtype=np.float32)
    kd = dev_f32(flat_k).as_strided((B, Hkv, nk, d), (0, nk * d // 2 + d, d // 2, 1))
    vd = dev_f32(flat_v).as_strided((B, Hkv, nk, d), (0, d, 0, 1))
    k = kd.cpu().numpy().astype(np.float64)
    v = vd.cpu().numpy().astype(np.float64)
    ref_o, ref_l = oracle.attention_fp64(q.astype(np.float64), k, v, causal=True, q_pos0=40)
    o, lse = _out(B, Hq, nq, d, torch.float32)
    api.ra_chunk_attention(dev_f32(q), kd, vd, o, lse, causal=True, q_pos0=40)
    torch.cuda.synchronize()
    check_close(host_f64(o), ref_o, "f32", "O")
    check_close(host_f64(lse).reshape(ref_l.shape), ref_l, "f32", "lse")
    # the bf16 kernel copies rows x row stride bytes: such views are refused
    with pytest.raises(api.SqkvError):
        api.ra_chunk_attention(dev_f32(q).bfloat16(), kd.bfloat16().as_strided((B, Hkv, nk, d), (0, 0, 0, 1)),
                               vd.bfloat16(), o, lse)


@pytest.mark.parametrize("Hq", [4, 256], ids=["split_kernel", "shared_kernel"])
def test_f32_inputs_bf16_state_and_output(api, Hq):
    """fp32 inputs merged into a bf16 running state, written as bf16: the
    merge reads bf16 rows and the epilogue rounds to bf16 (bf16 tolerance)."""
    B, Hkv, n, d = 1, 2, 150, 128
    say(f"f32 inputs, bf16 running state and output, Hq={Hq}")
    (q, k, v), (qd, kd, vd) = _inputs("f32", B, Hq, Hkv, n, 2 * n, d, seed=6400)
    ref_o, ref_l = oracle.attention_fp64(q, k, v, causal=True, q_pos0=n, k_pos0=0)
    o1, l1 = _out(B, Hq, n, d, torch.bfloat16)
    api.ra_chunk_attention(qd, kd[:, :, :n], vd[:, :, :n], o1, l1, causal=True, q_pos0=n, k_pos0=0)
    o2, l2 = _out(B, Hq, n, d, torch.bfloat16)
    api.ra_chunk_attention(qd, kd[:, :, n:], vd[:, :, n:], o2, l2, o_in=o1, lse_in=l1, causal=True,
                           q_pos0=n, k_pos0=n)
    torch.cuda.synchronize()
    check_close(host_f64(o2), ref_o, "bf16", "merged O")
    check_close(host_f64(l2).reshape(ref_l.shape), ref_l, "bf16", "merged lse")


def test_one_key_row_with_any_stride(api):
    """A one-row key/value view's row stride is never used: bf16 views with
    row stride 0 go through the binding and match the oracle."""
    B, Hq, Hkv, nq, d = 1, 4, 2, 70, 128
    say("bf16, one key with a stride-0 row view")
    (q, k, v), (qd, kd, vd) = _inputs("bf16", B, Hq, Hkv, nq, 1, d, seed=6300)
    kx = kd.as_strided((B, Hkv, 1, d), (kd.stride(0), kd.stride(1), 0, 1))
    vx = vd.as_strided((B, Hkv, 1, d), (vd.stride(0), vd.stride(1), 0, 1))
    assert kx.stride(2) == 0 and vx.stride(2) == 0
    ref_o, ref_l = oracle.attention_fp64(q, k, v)
    o, lse = _out(B, Hq, nq, d, torch.bfloat16)
    api.ra_chunk_attention(qd, kx, vx, o, lse)
    torch.cuda.synchronize()
    check_close(host_f64(o), ref_o, "bf16", "O")
    check_close(host_f64(lse).reshape(ref_l.shape), ref_l, "bf16", "lse")


# fp32 launches with at least one 128-row workgroup per compute unit (256 on
# MI355X) take the shared-tile kernel: these shapes have 256 or more
F32_WIDE_CASES = [
    # B, Hq, Hkv, nq, nk, d, causal, q_pos0, k_pos0
    (1, 256, 32, 130, 333, 128, True, 200, 0),    # ragged q-tile, causal diagonal, GQA 8:1
    (2, 128, 128, 257, 65, 64, False, 0, 0),      # three q-tiles; 3 key tiles (split 1 gets one)
    (1, 256, 256, 128, 1, 128, False, 0, 0),      # one key: split 1 has no tile at all
    (1, 256, 64, 100, 300, 64, True, 0, 150),     # rows before every key see nothing
]


@pytest.mark.parametrize("case", F32_WIDE_CASES, ids=_ids([c + (1.0,) for c in F32_WIDE_CASES]))
def test_f32_shared_kernel(api, case):
    B, Hq, Hkv, nq, nk, d, causal, qp, kp = case
    say(f"f32 shared-tile kernel {case}")
    (q, k, v), (qd, kd, vd) = _inputs("f32", B, Hq, Hkv, nq, nk, d, seed=7000 + nq + nk)
    ref_o, ref_l = oracle.attention_fp64(q, k, v, causal=causal, q_pos0=qp, k_pos0=kp)
    o, lse = _out(B, Hq, nq, d, torch.float32)
    api.ra_chunk_attention(qd, kd, vd, o, lse, causal=causal, q_pos0=qp, k_pos0=kp)
    torch.cuda.synchronize()
    check_close(host_f64(o), ref_o, "f32", "O")
    check_close(host_f64(lse).reshape(ref_l.shape), ref_l, "f32", "lse")


@pytest.mark.parametrize("d", [64, 128])
def test_f32_shared_kernel_accumulate_and_ring(api, d):
    """The shared-tile fp32 kernel with a running state (fused merge, in
    place) and over a causal ring of three chunks (every rank)."""
    B, Hq, Hkv, n = 1, 256, 32, 140
    say("f32 shared-tile kernel: fused merge")
    (q, k, v), (qd, kd, vd) = _inputs("f32", B, Hq, Hkv, n, 2 * n, d, seed=7100)
    ref_o, ref_l = oracle.attention_fp64(q, k, v, causal=True, q_pos0=n, k_pos0=0)
    o, lse = _out(B, Hq, n, d, torch.float32)
    api.ra_chunk_attention(qd, kd[:, :, :n], vd[:, :, :n], o, lse, causal=True, q_pos0=n, k_pos0=0)
    api.ra_chunk_attention(qd, kd[:, :, n:], vd[:, :, n:], o, lse, o_in=o, lse_in=lse, causal=True,
                           q_pos0=n, k_pos0=n)
    torch.cuda.synchronize()
    check_close(host_f64(o), ref_o, "f32", "merged O")
    check_close(host_f64(lse).reshape(ref_l.shape), ref_l, "f32", "merged lse")

    P, n = 3, 96
    say("f32 shared-tile kernel: causal ring of 3 chunks")
    pool = [_rand((P, B, Hq if i == 0 else Hkv, n, d), 7200 + i, d ** -0.5 if i == 0 else 1.0) for i in range(3)]
    ref_o, ref_l = oracle.attention_fp64(*[_full(x, "f32") for x in pool], causal=True)
    kp, vp = dev_f32(pool[1]), dev_f32(pool[2])
    for r in range(P):
        o, lse = _out(B, Hq, n, d, torch.float32)
        api.ra_ring_attention(dev_f32(pool[0][r]), kp, vp, o, lse, rank=r, scale=1.0, causal=True)
        torch.cuda.synchronize()
        check_close(host_f64(o), ref_o[:, :, r * n:(r + 1) * n], "f32", f"O rank {r}")
        check_close(host_f64(lse).reshape(B, Hq, n), ref_l[:, :, r * n:(r + 1) * n], "f32", f"lse rank {r}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_chunk_many_items_ragged_gqa(api, causal, d):
    """More (b, h, q-tile) items than CUs (several visits per workgroup) with
    item counts that fill neither the 8 XCDs evenly nor whole GQA groups of
    8*group, a ragged last q-tile and 5:1 GQA: every output written once
    (NaN-initialised, all finite) and equal to the oracle."""
    B, Hq, Hkv, nq, nk = 1, 150, 30, 520, 390
    say(f"chunk, {Hq} heads x 3 q-tiles, causal={causal}, d={d}")
    (q, k, v), (qd, kd, vd) = _inputs("bf16", B, Hq, Hkv, nq, nk, d, seed=900 + d + causal)
    ref_o, ref_l = oracle.attention_fp64(q, k, v, causal=causal, q_pos0=130 if causal else 0)
    o, lse = _out(B, Hq, nq, d, torch.bfloat16)
    api.ra_chunk_attention(qd, kd, vd, o, lse, causal=causal, q_pos0=130 if causal else 0)
    torch.cuda.synchronize()
    go, gl = host_f64(o), host_f64(lse).reshape(ref_l.shape)
    assert np.isfinite(go).all() and np.isfinite(gl).all(), "unwritten or non-finite outputs"
    check_close(go, ref_o, "bf16", "O")
    check_close(gl, ref_l, "bf16", "lse")


@pytest.mark.parametrize("in_dt", ["f32", "bf16"])
@pytest.mark.parametrize("inplace", [True, False])
def test_chunk_accumulate(api, in_dt, inplace):
    """Fused merge: (o_in, lse_in) from one key range, then a second chunk merged in."""
    B, Hq, Hkv, n, d = 1, 4, 2, 300, 128
    say(f"chunk accumulate {in_dt} inplace={inplace}")
    (q, k, v), (qd, kd, vd) = _inputs(in_dt, B, Hq, Hkv, n, 2 * n, d, seed=5)
    ref_o, ref_l = oracle.attention_fp64(q, k, v, causal=True, q_pos0=n, k_pos0=0)
    o1, l1 = _out(B, Hq, n, d, torch.float32)
    # first chunk: keys 0..n-1 (fully visible), second: keys n..2n-1 (diagonal)
    api.ra_chunk_attention(qd, kd[:, :, :n], vd[:, :, :n], o1, l1, causal=True, q_pos0=n, k_pos0=0)
    if inplace:
        o2, l2 = o1, l1
    else:
        o2, l2 = _out(B, Hq, n, d, torch.float32)
    api.ra_chunk_attention(qd, kd[:, :, n:], vd[:, :, n:], o2, l2, o_in=o1, lse_in=l1, causal=True,
                           q_pos0=n, k_pos0=n)
    torch.cuda.synchronize()
    tol = "bf16" if in_dt == "bf16" else "f32"
    check_close(host_f64(o2), ref_o, tol, "merged O")
    check_close(host_f64(l2).reshape(ref_l.shape), ref_l, tol, "merged lse")


@pytest.mark.parametrize("in_dt,Hq", [("f32", 4), ("f32", 256), ("bf16", 4)],
                         ids=["f32-split_kernel", "f32-shared_kernel", "bf16"])
def test_empty_key_chunk(api, in_dt, Hq):
    """A chunk with no keys (n_k = 0, key/value tensors with no rows): its own
    partial is O = 0, lse = -inf, and merged into a running result it leaves
    that result as it was.  No key or value memory is read."""
    B, Hkv, n, d = 1, 2, 130, 128
    say(f"empty key chunk {in_dt} Hq={Hq}")
    (q, k, v), (qd, kd, vd) = _inputs(in_dt, B, Hq, Hkv, n, 200, d, seed=21)
    ke, ve = kd[:, :, :0], vd[:, :, :0]
    ref_e, ref_le = oracle.attention_fp64(q, k[:, :, :0], v[:, :, :0])
    o, lse = _out(B, Hq, n, d, torch.float32)
    api.ra_chunk_attention(qd, ke, ve, o, lse)
    torch.cuda.synchronize()
    tol = "bf16" if in_dt == "bf16" else "f32"
    check_close(host_f64(o), ref_e, tol, "empty partial O")
    check_close(host_f64(lse).reshape(ref_le.shape), ref_le, tol, "empty partial lse")
    # a running result from 200 real keys, then the empty chunk merged in
    o1, l1 = _out(B, Hq, n, d, torch.float32)
    api.ra_chunk_attention(qd, kd, vd, o1, l1)
    o2, l2 = _out(B, Hq, n, d, torch.float32)
    api.ra_chunk_attention(qd, ke, ve, o2, l2, o_in=o1, lse_in=l1)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.lse_merge_fp64(host_f64(o1), host_f64(l1).reshape(ref_le.shape), ref_e, ref_le)
    check_close(host_f64(o2), ref_o, tol, "merged O")
    check_close(host_f64(l2).reshape(ref_l.shape), ref_l, tol, "merged lse")


@pytest.mark.parametrize("in_dt,Hq", [("f32", 2), ("f32", 160), ("bf16", 2)],
                         ids=["f32-split_kernel", "f32-shared_kernel", "bf16"])
def test_running_max_rescale(api, in_dt, Hq):
    """Keys that grow along the sequence force the running maximum up tile after tile.

    With 160 heads of two 128-row query tiles the fp32 launch has 320
    workgroups and takes the shared-tile kernel; with 2 heads, the split one."""
    B, n, d = 1, 256, 64
    say(f"rescale path {in_dt} Hq={Hq}")
    (q, k, v), (qd, kd, vd) = _inputs(in_dt, B, Hq, Hq, n, 1000, d, seed=9, qscale=0.5, kramp=True)
    ref_o, ref_l = oracle.attention_fp64(q, k, v, scale=1.0)
    o, lse = _out(B, Hq, n, d, torch.float32)
    api.ra_chunk_attention(qd, kd, vd, o, lse, scale=1.0)
    torch.cuda.synchronize()
    tol = "bf16" if in_dt == "bf16" else "f32"
    check_close(host_f64(o), ref_o, tol, "O")
    got_l = host_f64(lse).reshape(ref_l.shape)
    if in_dt == "bf16":
        check_close(got_l, ref_l, "bf16", "lse")        # 2e-2 max-abs, with lse reaching O(100)
    else:
        assert np.max(np.abs(got_l - ref_l) / np.maximum(np.abs(ref_l), 1.0)) < 1e-5


def _extreme_inputs(B, H, nq, nk, d, seed, kind):
    """bf16 inputs whose base-2 scores leave float's range without a shift.

    Every key and query shares a large common direction u, so every score of a
    row is far from zero whatever the mask: "overflow" puts them near +384
    (nats), "underflow" near -256, both with a spread of a few nats from the
    rest; "mixed" is overflow on even heads and ordinary scores on odd heads
    (workgroups of one launch take different passes)."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, nq, d), dtype=np.float32)
    k = rng.standard_normal((B, H, nk, d), dtype=np.float32)
    v = rng.standard_normal((B, H, nk, d), dtype=np.float32)
    u = rng.standard_normal((B, H, 1, d), dtype=np.float32)
    if kind == "underflow":
        q, k = np.float32(-2.0) * u + np.float32(0.1) * q, u + np.float32(0.1) * k
    else:
        qx, kx = np.float32(3.0) * u + np.float32(0.3) * q, u + np.float32(0.3) * k
        if kind == "mixed":
            qx[:, 1::2] = q[:, 1::2] / np.float32(math.sqrt(d))
            kx[:, 1::2] = k[:, 1::2]
        q, k = qx, kx
    bits = [f32_to_bf16_bits(x) for x in (q, k, v)]
    return [bf16_bits_to_f64(b) for b in bits], [dev_bf16(b) for b in bits]


def _check_extreme(o, lse, ref_o, ref_l, what):
    check_close(host_f64(o), ref_o, "bf16", f"{what} O")
    check_close(host_f64(lse).reshape(ref_l.shape), ref_l, "bf16", f"{what} lse")


@pytest.mark.parametrize("kind", ["overflow", "underflow", "mixed"])
@pytest.mark.parametrize("causal", [False, True])
def test_fast_pass_fallback(api, kind, causal):
    """Scores whose exponentials leave float's range without a shift: the
    workgroups concerned redo the visit with the running maximum."""
    B, H, nq, nk, d = 1, 4, 520, 600, 128
    say(f"fast-pass fallback {kind} causal={causal}")
    (q, k, v), (qd, kd, vd) = _extreme_inputs(B, H, nq, nk, d, seed=31, kind=kind)
    ref_o, ref_l = oracle.attention_fp64(q, k, v, scale=1.0, causal=causal, q_pos0=nk - nq)
    o, lse = _out(B, H, nq, d, torch.float32)
    api.ra_chunk_attention(qd, kd, vd, o, lse, scale=1.0, causal=causal, q_pos0=nk - nq)
    torch.cuda.synchronize()
    _check_extreme(o, lse, ref_o, ref_l, kind)


def test_fast_pass_fallback_ring(api):
    """The fallback over a ring visit of three chunks (the walkers restart)."""
    P, B, H, n, d = 3, 1, 2, 300, 128
    say("fast-pass fallback ring")
    (q, k, v), (qd, kd, vd) = _extreme_inputs(B, H, P * n, P * n, d, seed=33, kind="mixed")
    ref_o, ref_l = oracle.attention_fp64(q, k, v, scale=1.0, causal=True)
    pool = lambda x: x.reshape(B, H, P, n, d).permute(2, 0, 1, 3, 4).contiguous()
    kp, vp = pool(kd), pool(vd)
    for i in range(P):
        o, lse = _out(B, H, n, d, torch.bfloat16)
        api.ra_ring_attention(qd[:, :, i * n:(i + 1) * n].contiguous(), kp, vp, o, lse, rank=i, scale=1.0,
                              causal=True)
        torch.cuda.synchronize()
        sl = slice(i * n, (i + 1) * n)
        _check_extreme(o, lse, ref_o[:, :, sl], ref_l[:, :, sl], f"rank {i}")


def _edge_inputs(B, H, nq, nk, d, seed):
    from sequence_kv_chunk_amd.synth import aligned_score_inputs
    bits = aligned_score_inputs(B, H, nq, nk, d, seed)
    return [bf16_bits_to_f64(b) for b in bits], [dev_bf16(b) for b in bits]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_fast_pass_rounding_edge(api, d, causal):
    """Scores of 9-17 nats on every key, all aligned with the query, row sums
    2^20-2^36 (inside the window where the fast pass keeps its result), and
    query elements chosen so that a rescaled-and-re-rounded Q would move every
    score the same way: O and lse within the bar, fp32 and bf16 outputs."""
    B, H, nq, nk = 1, 4, 300, 2048
    say(f"fast-pass rounding edge d={d} causal={causal}")
    (q, k, v), (qd, kd, vd) = _edge_inputs(B, H, nq, nk, d, seed=50 + d + int(causal))
    qp = nk - nq if causal else 0
    ref_o, ref_l = oracle.attention_fp64(q, k, v, scale=1.0, causal=causal, q_pos0=qp)
    for odt in (torch.float32, torch.bfloat16):
        o, lse = _out(B, H, nq, d, odt)
        api.ra_chunk_attention(qd, kd, vd, o, lse, scale=1.0, causal=causal, q_pos0=qp)
        torch.cuda.synchronize()
        eo = check_close(host_f64(o), ref_o, "bf16", f"O {odt}")
        el = check_close(host_f64(lse).reshape(ref_l.shape), ref_l, "bf16", "lse")
        say(f"   out {odt}: O err {eo:.2e}, lse err {el:.2e}")


def test_rounding_edge_unfused_merge(api):
    """The same inputs over two key ranges, each written out as an fp32 partial
    and merged by ra_lse_merge (the merge weights come from the partials' lse)."""
    B, H, nq, nk, d = 1, 4, 300, 2048, 128
    say("rounding edge, unfused merge")
    (q, k, v), (qd, kd, vd) = _edge_inputs(B, H, nq, nk, d, seed=61)
    ref_o, ref_l = oracle.attention_fp64(q, k, v, scale=1.0)
    half = 1000                                  # not a multiple of the key tile
    parts = []
    for sl in (slice(0, half), slice(half, nk)):
        o, lse = _out(B, H, nq, d, torch.float32)
        api.ra_chunk_attention(qd, kd[:, :, sl].contiguous(), vd[:, :, sl].contiguous(), o, lse, scale=1.0)
        parts.append((o, lse))
    for odt in (torch.float32, torch.bfloat16):
        o, lse = _out(B, H, nq, d, odt)
        api.ra_lse_merge(parts[0][0], parts[0][1], parts[1][0], parts[1][1], o, lse)
        torch.cuda.synchronize()
        check_close(host_f64(o), ref_o, "bf16", f"merged O {odt}")
        check_close(host_f64(lse).reshape(ref_l.shape), ref_l, "bf16", "merged lse")


@pytest.mark.parametrize("split", ["ring", "zigzag"])
def test_rounding_edge_causal_ring(api, split):
    """A causal ring of 4 ranks on the same inputs, contiguous chunks (one
    launch per rank) and the zigzag split (three launches per rank, the last
    merging with the second's partial)."""
    P, B, H, n, d = 4, 1, 4, 512, 128
    L = P * n
    say(f"rounding edge, causal {split}")
    from sequence_kv_chunk_amd.synth import aligned_score_inputs
    qb, kb, vb = aligned_score_inputs(B, H, L, L, d, seed=70)
    q, k, v = (bf16_bits_to_f64(b) for b in (qb, kb, vb))
    if split == "ring":
        pos = [np.arange(r * n, (r + 1) * n) for r in range(P)]
    else:
        pos = [oracle.zigzag_positions(r, P, n // 2) for r in range(P)]
    shard = lambda bits: np.stack([bits[:, :, p] for p in pos])          # [P, B, H, n, d]
    qs, kp, vp = dev_bf16(shard(qb)), dev_bf16(shard(kb)), dev_bf16(shard(vb))
    ref_o, ref_l = oracle.attention_fp64(q, k, v, scale=1.0, causal=True)
    for r in range(P):
        o, lse = _out(B, H, n, d, torch.bfloat16)
        if split == "ring":
            api.ra_ring_attention(qs[r], kp, vp, o, lse, rank=r, scale=1.0, causal=True)
        else:
            work = (torch.empty((B, H, n // 2, d), dtype=torch.float32, device="cuda"),
                    torch.empty(B * H * (n // 2), dtype=torch.float32, device="cuda"))
            api.ra_zigzag_attention(qs[r], kp, vp, o, lse, rank=r, scale=1.0, work=work)
        torch.cuda.synchronize()
        check_close(host_f64(o), ref_o[:, :, pos[r]], "bf16", f"O rank {r}")
        check_close(host_f64(lse).reshape(B, H, n), ref_l[:, :, pos[r]], "bf16", f"lse rank {r}")


def test_shd_layout_gqa(api):
    """A Ulysses share in its natural [S, H, d] layout (strided views), GQA 4:1, causal."""
    S, Hq, Hkv, d = 700, 4, 1, 128
    say("shd layout")
    rng = np.random.default_rng(11)
    q = f32_to_bf16_bits(rng.standard_normal((S, Hq, d), dtype=np.float32) / np.float32(math.sqrt(d)))
    k = f32_to_bf16_bits(rng.standard_normal((S, Hkv, d), dtype=np.float32))
    v = f32_to_bf16_bits(rng.standard_normal((S, Hkv, d), dtype=np.float32))
    to_bhnd = lambda x: bf16_bits_to_f64(x).transpose(1, 0, 2)[None]
    ref_o, ref_l = oracle.attention_fp64(to_bhnd(q), to_bhnd(k), to_bhnd(v), causal=True)
    o = torch.full((S, Hq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(Hq * S, dtype=torch.float32, device="cuda")
    api.ra_chunk_attention(dev_bf16(q), dev_bf16(k), dev_bf16(v), o, lse, causal=True)
    torch.cuda.synchronize()
    check_close(host_f64(o).transpose(1, 0, 2)[None], ref_o, "bf16", "O [S,H,d]")
    check_close(host_f64(lse).reshape(ref_l.shape), ref_l, "bf16", "lse")


def _ring_run(api, w, qb, kb, vb, ranks, L=None, P=None):
    """Runs ra_ring_attention for the given ranks; returns host O (f64) and lse."""
    P = w.P if P is None else P
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dev = dev_bf16 if w.dtype == "bf16" else dev_f32
    kp, vp = dev(kb), dev(vb)
    outs = []
    for idx, i in enumerate(ranks):
        qi = dev(qb[idx])
        B, H, n, d = qi.shape
        o, lse = _out(B, H, n, d, dt)
        api.ra_ring_attention(qi, kp, vp, o, lse, rank=i, scale=1.0, causal=w.causal)
        torch.cuda.synchronize()
        outs.append((host_f64(o), host_f64(lse).reshape(B, H, n)))
    return outs


def _full(x, dtype):
    """Pool [P, B, H, n, d] -> whole sequence [B, H, P*n, d] as float64."""
    x = bf16_bits_to_f64(x) if dtype == "bf16" else x.astype(np.float64)
    P, B, H, n, d = x.shape
    return x.transpose(1, 2, 0, 3, 4).reshape(B, H, P * n, d)


def test_ring_f32_tiny(api):
    """Four virtual ranks, 1024 tokens as 4 chunks of 256, fp32: equals full softmax."""
    w = WORKLOADS["ring_f32_tiny"]
    say(f"ring {w.name}")
    x = attention_inputs(w)
    ref_o, ref_l = oracle.attention_fp64(_full(x["q"], "f32"), _full(x["k"], "f32"), _full(x["v"], "f32"))
    outs = _ring_run(api, w, x["q"], x["k"], x["v"], range(w.P))
    n = w.n
    for i, (o, l) in enumerate(outs):
        check_close(o, ref_o[:, :, i * n:(i + 1) * n], "f32", f"O rank {i}")
        check_close(l, ref_l[:, :, i * n:(i + 1) * n], "f32", f"lse rank {i}")


@pytest.mark.parametrize("causal", [False, True])
def test_chunk_f32_4k_sampled(api, causal):
    """The exact fp32 path at the size bench.py times (one 4096 x 4096 chunk
    pair, 32 heads, d=128; also causal): every output finite, and sampled
    rows of four heads (the first and last row of every 32-row workgroup
    among them) against the fp64 oracle at the fp32 bar."""
    B, H, n, d = 1, 32, 4096, 128
    say(f"fp32 chunk 4k causal={causal}")
    rng = np.random.default_rng(4096 + int(causal))
    q = rng.standard_normal((B, H, n, d), dtype=np.float32) * np.float32(d ** -0.5)
    k = rng.standard_normal((B, H, n, d), dtype=np.float32)
    v = rng.standard_normal((B, H, n, d), dtype=np.float32)
    o = torch.full((B, H, n, d), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((B * H * n,), float("nan"), dtype=torch.float32, device="cuda")
    api.ra_chunk_attention(dev_f32(q), dev_f32(k), dev_f32(v), o, lse, causal=causal)
    torch.cuda.synchronize()
    og, lg = host_f64(o), host_f64(lse).reshape(B, H, n)
    assert np.isfinite(og).all() and np.isfinite(lg).all()
    heads = [0, 9, 22, H - 1]
    # first and last row of every 32-row workgroup, and every 97th row
    rows = np.array(sorted({*range(0, n, 32), *range(31, n, 32), *range(5, n, 97), n - 1}), dtype=np.int64)
    qf, kf, vf = q[:, heads][:, :, rows], k[:, heads], v[:, heads]
    if causal:
        ref_o, ref_l = oracle.attention_at_positions_fp64(qf, kf, vf, rows, np.arange(n))
    else:
        ref_o, ref_l = oracle.attention_fp64(qf, kf, vf)
    check_close(og[:, heads][:, :, rows], ref_o, "f32", "O sampled rows")
    check_close(lg[:, heads][:, :, rows], ref_l, "f32", "lse sampled rows")
    say(f"   {len(rows)} rows x {len(heads)} heads checked")


def test_ring_f32_tiny_unfused_merge(api):
    """The same ring with each chunk's partial written out and merged by ra_lse_merge."""
    w = WORKLOADS["ring_f32_tiny"]
    x = attention_inputs(w)
    ref_o, ref_l = oracle.attention_fp64(_full(x["q"], "f32"), _full(x["k"], "f32"), _full(x["v"], "f32"))
    kp, vp = dev_f32(x["k"]), dev_f32(x["v"])
    n = w.n
    for i in range(w.P):
        qi = dev_f32(x["q"][i])
        acc_o, acc_l = _out(1, w.Hq, n, w.d, torch.float32)
        part_o, part_l = _out(1, w.Hq, n, w.d, torch.float32)
        for s in range(w.P):
            j = (i - s) % w.P
            tgt = (acc_o, acc_l) if s == 0 else (part_o, part_l)
            api.ra_chunk_attention(qi, kp[j], vp[j], *tgt, q_pos0=i * n, k_pos0=j * n)
            if s > 0:
                api.ra_lse_merge(acc_o, acc_l, part_o, part_l, acc_o, acc_l)
        torch.cuda.synchronize()
        check_close(host_f64(acc_o), ref_o[:, :, i * n:(i + 1) * n], "f32", f"O rank {i}")
        check_close(host_f64(acc_l).reshape(1, w.Hq, n), ref_l[:, :, i * n:(i + 1) * n], "f32", "lse")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("P", [1, 2, 3, 8])
def test_ring_bf16_small(api, P, causal):
    """The bf16 32k ring in miniature: 8 chunks of 256 tokens (and other P), all ranks."""
    base = WORKLOADS["ring_bf16_32k"]
    L = 256 * P
    import dataclasses
    w = dataclasses.replace(base, L=L, P=P, Hq=4, Hkv=4, causal=causal)
    say(f"ring bf16 small P={P} causal={causal}")
    x = attention_inputs(w)
    ref_o, ref_l = oracle.attention_fp64(_full(x["q"], "bf16"), _full(x["k"], "bf16"), _full(x["v"], "bf16"),
                                         causal=causal)
    outs = _ring_run(api, w, x["q"], x["k"], x["v"], range(P))
    n = w.n
    for i, (o, l) in enumerate(outs):
        check_close(o, ref_o[:, :, i * n:(i + 1) * n], "bf16", f"O rank {i}")
        check_close(l, ref_l[:, :, i * n:(i + 1) * n], "bf16", f"lse rank {i}")


@pytest.mark.parametrize("in_dt,Hq", [("bf16", 8), ("f32", 8), ("f32", 256)],
                         ids=["bf16", "f32_split_kernel", "f32_shared_kernel"])
def test_deterministic(api, in_dt, Hq):
    """Two runs of the same call give bitwise the same outputs (no atomics,
    a fixed merge order of the key splits)."""
    (q, k, v), (qd, kd, vd) = _inputs(in_dt, 1, Hq, 2, 700, 900, 128, seed=21)
    res = []
    for _ in range(2):
        o, lse = _out(1, Hq, 700, 128, torch.float32)
        api.ra_chunk_attention(qd, kd, vd, o, lse, causal=True, q_pos0=300)
        torch.cuda.synchronize()
        res.append((o.cpu().numpy().tobytes(), lse.cpu().numpy().tobytes()))
    assert res[0] == res[1], "two runs differ bitwise"


# ---------------------------------------------------------------------------
# full-size workloads, sampled rows
# ---------------------------------------------------------------------------
QTILE = 256      # query rows per workgroup of the bf16 kernel


def _tile_edge_rows(n, rng, extra):
    """Rows 0..n-1 of one query chunk to check: the first and last row of every
    256-row query tile (so also of the chunk) plus `extra` random rows."""
    rows = {0, n - 1}
    for t0 in range(0, n, QTILE):
        rows.update((t0, min(n, t0 + QTILE) - 1))
    rows.update(int(r) for r in rng.integers(0, n, size=extra))
    return np.array(sorted(rows), dtype=np.int64)


def _all_finite(o, lse, what):
    """Every element of a full-size output was written (the buffers start as
    NaN) and is finite."""
    assert np.isfinite(o).all(), f"{what}: O holds non-finite values (unwritten tiles?)"
    assert np.isfinite(lse).all(), f"{what}: lse holds non-finite values (unwritten rows?)"


def _check_rows_causal(o_rows, l_rows, q_rows, kf, vf, q_pos, what):
    """Sampled rows of one head against the oracle at explicit positions: q_rows
    [1, 1, r, d] bf16 bits, kf/vf [1, 1, L, d] float64 (keys at 0..L-1)."""
    ref_o, ref_l = oracle.attention_at_positions_fp64(bf16_bits_to_f64(q_rows), kf, vf, q_pos,
                                                      np.arange(kf.shape[2]))
    check_close(o_rows, ref_o, "bf16", f"O {what}")
    check_close(l_rows, ref_l, "bf16", f"lse {what}")
    return ref_o.shape[2]


@pytest.mark.slow
def test_ring_bf16_32k_full(api):
    """The whole 32k ring (8 ranks x 8 chunks of 4096, 32 heads), the launch
    sequence bench.py times: every output element finite, and in every head of
    every rank the first and last row of each 256-row query tile plus random
    rows against one softmax over all 32768 keys (9000+ rows)."""
    w = WORKLOADS["ring_bf16_32k"]
    say(f"full size {w.name}")
    x = attention_inputs(w)
    outs = _ring_run(api, w, x["q"], x["k"], x["v"], range(w.P))
    for i, (o, l) in enumerate(outs):
        _all_finite(o, l, f"rank {i}")
    rng = np.random.default_rng(123)
    n, checked = w.n, 0
    for h in range(w.Hq):
        kf = _full(x["k"][:, :, h:h + 1], "bf16")
        vf = _full(x["v"][:, :, h:h + 1], "bf16")
        for i, (o, l) in enumerate(outs):
            rows = _tile_edge_rows(n, rng, extra=4)
            ref_o, ref_l = oracle.attention_fp64(bf16_bits_to_f64(x["q"][i][:, h:h + 1, rows]), kf, vf)
            check_close(o[:, h:h + 1, rows], ref_o, "bf16", f"O rank {i} head {h}")
            check_close(l[:, h:h + 1, rows], ref_l, "bf16", f"lse rank {i} head {h}")
            checked += rows.size
    say(f"   {checked} rows checked")
    assert checked >= 2048


@pytest.mark.slow
def test_ring_128k_rank7_causal_full(api):
    """Rank 7 of the causal 128k ring (chunk of 16384 against 8 chunks, 32
    heads): every output element finite, and in every head the first and last
    row of each 256-row query tile plus random rows against the causal softmax
    over the 114689..131072 keys each row sees (4000+ rows)."""
    w = WORKLOADS["ring_bf16_128k_rank7_causal"]
    say(f"full size {w.name}")
    x = attention_inputs(w)
    (o, l), = _ring_run(api, w, x["q"], x["k"], x["v"], w.query_ranks)
    _all_finite(o, l, "rank 7")
    rng = np.random.default_rng(7)
    n, rank, checked = w.n, w.query_ranks[0], 0
    for h in range(w.Hq):
        kf = _full(x["k"][:, :, h:h + 1], "bf16")
        vf = _full(x["v"][:, :, h:h + 1], "bf16")
        rows = _tile_edge_rows(n, rng, extra=8)
        checked += _check_rows_causal(o[:, h:h + 1, rows], l[:, h:h + 1, rows], x["q"][0][:, h:h + 1, rows],
                                      kf, vf, rank * n + rows, f"head {h}")
    say(f"   {checked} rows checked")
    assert checked >= 2048


@pytest.mark.slow
def test_ulysses_share_gqa_128k_full(api):
    """One Ulysses share: causal attention over 131072 tokens, 4 query heads on
    1 key/value head, [S, H, d] layout: every output element finite, no L x L
    allocation, and in every head the first and last row of each 256-row query
    tile plus random rows against the oracle (4000+ rows)."""
    w = WORKLOADS["ulysses_share_gqa_128k_causal"]
    say(f"full size {w.name}")
    x = attention_inputs(w)
    qd, kd, vd = dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"])
    free0 = torch.cuda.mem_get_info()[0]
    o = torch.full((w.L, w.Hq, w.d), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((w.Hq * w.L,), float("nan"), dtype=torch.float32, device="cuda")
    api.ra_chunk_attention(qd, kd, vd, o, lse, causal=True)
    torch.cuda.synchronize()
    # the library allocates nothing: no L x L score matrix (32 GiB per head at this length)
    assert free0 - torch.cuda.mem_get_info()[0] < oracle.attn_matrix_bytes(w.L) // 64
    oh = host_f64(o)                                   # [L, Hq, d]
    lh = host_f64(lse).reshape(w.Hq, w.L)
    del qd, kd, vd, o, lse
    _all_finite(oh, lh, "share")
    kf = bf16_bits_to_f64(x["k"]).transpose(1, 0, 2)[None]
    vf = bf16_bits_to_f64(x["v"]).transpose(1, 0, 2)[None]
    rng = np.random.default_rng(5)
    checked = 0
    for h in range(w.Hq):
        rows = _tile_edge_rows(w.L, rng, extra=16)
        q_rows = x["q"][rows, h:h + 1].transpose(1, 0, 2)[None]                 # [1, 1, r, d]
        checked += _check_rows_causal(oh[rows, h:h + 1].transpose(1, 0, 2)[None], lh[h:h + 1, rows][None],
                                      q_rows, kf, vf, rows, f"head {h}")
    say(f"   {checked} rows checked")
    assert checked >= 2048


@pytest.mark.slow
def test_causal_1m_tokens_sampled(api):
    """Capacity: causal attention over 1,048,576 tokens in one call (4 query
    heads, 1 key/value head, d=128), with no L x L allocation (2 TiB per head
    at this length); sampled rows against the oracle."""
    L, Hq, Hkv, d = 1 << 20, 4, 1, 128
    say(f"causal attention over {L} tokens")
    rng = np.random.default_rng(11)
    qb = f32_to_bf16_bits(rng.standard_normal((L, Hq, d), dtype=np.float32) * np.float32(d ** -0.5))
    kb = f32_to_bf16_bits(rng.standard_normal((L, Hkv, d), dtype=np.float32))
    vb = f32_to_bf16_bits(rng.standard_normal((L, Hkv, d), dtype=np.float32))
    qd, kd, vd = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb)
    o = torch.full((L, Hq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(Hq * L, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    api.ra_chunk_attention(qd, kd, vd, o, lse, causal=True)
    torch.cuda.synchronize()
    # no L x L buffer (2 TiB per head here): the library allocates nothing, and
    # the bound leaves room for what the HIP runtime itself may reserve on a
    # kernel's first launch
    assert free0 - torch.cuda.mem_get_info()[0] < oracle.attn_matrix_bytes(L) // 4096
    # every element written (the output starts as NaN) and finite
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    rows = sorted({0, 1, 4095, L // 2 + 7, L - 1, *(int(i) for i in rng.integers(0, L, size=3))})
    oh = {r: host_f64(o[r:r + 1]) for r in rows}                      # [1, Hq, d] each
    lh = host_f64(lse).reshape(Hq, L)
    del qd, kd, vd, o, lse
    kf = bf16_bits_to_f64(kb).transpose(1, 0, 2)[None]
    vf = bf16_bits_to_f64(vb).transpose(1, 0, 2)[None]
    for r in rows:
        qh = bf16_bits_to_f64(qb[r:r + 1]).transpose(1, 0, 2)[None]
        ref_o, ref_l = oracle.attention_fp64(qh, kf[:, :, :r + 1], vf[:, :, :r + 1])
        check_close(oh[r].transpose(1, 0, 2)[None], ref_o, "bf16", f"O row {r}")
        check_close(lh[:, r:r + 1][None], ref_l, "bf16", f"lse row {r}")

"""Launches at the largest grid the library admits: B or Hq at 65535 (the
limit that the host validation states, set by the grid's y and z
dimensions), with a few rows per head.  Every output is checked for
finiteness on the device; sampled heads (the first and last eight and 32 in
between) are checked against the oracle at the usual tolerances."""
import numpy as np
import pytest

import oracle
from sequence_kv_chunk_amd.synth import bf16_bits_to_f64, f32_to_bf16_bits

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from gpu_util import check_close, dev_bf16, dev_f32, host_f64, say  # noqa: E402
from test_gpu_backward import check_grad  # noqa: E402


@pytest.fixture(scope="module")
def api():
    from sequence_kv_chunk_amd import api
    return api


def _heads(B, H, seed):
    """(b, h) pairs: the first and last eight of the B*H heads and 32 between."""
    n = B * H
    rng = np.random.default_rng(seed)
    flat = np.unique(np.concatenate([np.arange(8), np.arange(n - 8, n), rng.integers(8, n - 8, 32)]))
    return [(int(i // H), int(i % H)) for i in flat]


def _tensor(shape, rng, dtype, scale=1.0):
    x = rng.standard_normal(shape, dtype=np.float32) * np.float32(scale)
    if dtype == "bf16":
        bits = f32_to_bf16_bits(x)
        return bf16_bits_to_f64(bits), dev_bf16(bits)
    return x.astype(np.float64), dev_f32(x)


LIMIT_CASES = [
    # B, Hq, Hkv, n_q, n_k, d
    (1, 65535, 5, 3, 5, 64),       # grid y at its limit, GQA 13107:1
    (65535, 2, 1, 3, 5, 64),       # grid z at its limit
]


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("case", LIMIT_CASES, ids=["Hq65535", "B65535"])
def test_forward_at_grid_limits(api, case, dt):
    B, Hq, Hkv, nq, nk, d = case
    say(f"forward at grid limits {case} {dt}")
    rng = np.random.default_rng(B + Hq)
    q, qd = _tensor((B, Hq, nq, d), rng, dt, d ** -0.5)
    k, kd = _tensor((B, Hkv, nk, d), rng, dt)
    v, vd = _tensor((B, Hkv, nk, d), rng, dt)
    o = torch.full((B, Hq, nq, d), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((B * Hq * nq,), float("nan"), dtype=torch.float32, device="cuda")
    api.ra_chunk_attention(qd, kd, vd, o, lse)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all()), "unwritten or non-finite outputs"
    got_o, got_l = host_f64(o), host_f64(lse).reshape(B, Hq, nq)
    group = Hq // Hkv
    for b, h in _heads(B, Hq, seed=nq + nk):
        g = h // group
        ref_o, ref_l = oracle.attention_fp64(q[b:b + 1, h:h + 1], k[b:b + 1, g:g + 1], v[b:b + 1, g:g + 1])
        check_close(got_o[b:b + 1, h:h + 1], ref_o, dt, f"O b={b} h={h}")
        check_close(got_l[b:b + 1, h:h + 1], ref_l, dt, f"lse b={b} h={h}")


@pytest.mark.parametrize("B,H", [(1, 65535), (65535, 1)], ids=["H65535", "B65535"])
def test_backward_at_grid_limits(api, B, H):
    nq, nk, d = 3, 5, 64
    say(f"backward at grid limits B={B} H={H}")
    rng = np.random.default_rng(B + 7 * H)
    q, qd = _tensor((B, H, nq, d), rng, "bf16", d ** -0.5)
    k, kd = _tensor((B, H, nk, d), rng, "bf16")
    v, vd = _tensor((B, H, nk, d), rng, "bf16")
    do, dod = _tensor((B, H, nq, d), rng, "bf16")
    ref_o, ref_l = oracle.attention_fp64(q, k, v)
    D = oracle.rowsum_do_o_fp64(do, ref_o)
    lse_d = dev_f32(ref_l.reshape(-1))
    D_d = dev_f32(D.reshape(-1))
    dq = torch.zeros((B, H, nq, d), dtype=torch.float32, device="cuda")
    dk = torch.zeros((B, H, nk, d), dtype=torch.float32, device="cuda")
    dv = torch.zeros((B, H, nk, d), dtype=torch.float32, device="cuda")
    api.ra_chunk_attention_bwd(qd, kd, vd, dod, lse_d, D_d, dq, dk, dv)
    torch.cuda.synchronize()
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert bool(torch.isfinite(t).all()), f"{name}: non-finite values"
    gq, gk, gv = host_f64(dq), host_f64(dk), host_f64(dv)
    for b, h in _heads(B, H, seed=11):
        s = (slice(b, b + 1), slice(h, h + 1))
        rq, rk, rv = oracle.chunk_attention_bwd_fp64(q[s], k[s], v[s], do[s], ref_l[s], D[s])
        check_grad(gq[s], rq, f"dq b={b} h={h}")
        check_grad(gk[s], rk, f"dk b={b} h={h}")
        check_grad(gv[s], rv, f"dv b={b} h={h}")

"""USP hybrid (usp_attention: Ulysses inside groups of P_u virtual ranks, ring
attention across the P_r groups) against one softmax over the whole sequence
in the fp64 oracle; covers pure ring (P_u = 1), pure Ulysses (P_r = 1) and
key/value head copying (P_u > H_kv)."""
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
    # P_u, P_r, L, H, H_kv, d, causal
    (2, 2, 1024, 4, 2, 128, False),
    (2, 2, 1024, 4, 2, 128, True),
    (4, 2, 2048, 8, 2, 64, True),      # H_kv < P_u: each KV head copied to 2 ranks
    (1, 4, 1024, 2, 1, 128, True),     # pure ring
    (4, 1, 1024, 8, 8, 128, True),     # pure Ulysses
    (2, 3, 1200, 4, 4, 128, False),    # ragged tiles (chunks of 400)
]


@pytest.mark.parametrize("case", CASES, ids=[f"u{c[0]}r{c[1]}_L{c[2]}_c{int(c[6])}" for c in CASES])
def test_usp(api, case):
    P_u, P_r, L, H, H_kv, d, causal = case
    say(f"usp {case}")
    P = P_u * P_r
    n = L // P
    rng = np.random.default_rng(3000 + L + P_u)
    qb = f32_to_bf16_bits(rng.standard_normal((P, n, H, d), dtype=np.float32) * np.float32(d ** -0.5))
    kb = f32_to_bf16_bits(rng.standard_normal((P, n, H_kv, d), dtype=np.float32))
    vb = f32_to_bf16_bits(rng.standard_normal((P, n, H_kv, d), dtype=np.float32))
    # natural order [1, H, L, d] for the oracle
    nat = lambda x: bf16_bits_to_f64(x).reshape(L, x.shape[2], d).transpose(1, 0, 2)[None]
    ref_o, ref_l = oracle.attention_fp64(nat(qb), nat(kb), nat(vb), causal=causal)
    o = torch.full((P, n, H, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = api.usp_attention(dev_bf16(qb), dev_bf16(kb), dev_bf16(vb), o, P_u=P_u, causal=causal)
    torch.cuda.synchronize()
    got_o = host_f64(o).reshape(L, H, d).transpose(1, 0, 2)[None]
    check_close(got_o, ref_o, "bf16", f"O {case}")
    # lse [P_r, P_u, H/P_u, S]: ring row i_r holds tokens i_r*S .., share i_u heads i_u*H/P_u ..
    S = L // P_r
    got_l = host_f64(lse).reshape(P_r, P_u, H // P_u, S).transpose(1, 2, 0, 3).reshape(H, L)[None]
    check_close(got_l, ref_l, "bf16", f"lse {case}")


@pytest.mark.slow
@pytest.mark.parametrize("P_u", [4, 2])
def test_usp_128k_full_sampled(api, P_u):
    """USP at the shape bench.py times (L = 131072, 32 query heads, 8 key/value
    heads, d = 128, 8 virtual ranks, causal): sampled tokens and heads against
    the oracle's softmax over each token's causal prefix."""
    L, H, H_kv, d, P = 131072, 32, 8, 128, 8
    n, S = L // P, L // (P // P_u)
    say(f"usp 128k full size, P_u={P_u}")
    rng = np.random.default_rng(4000 + P_u)
    qb = f32_to_bf16_bits(rng.standard_normal((P, n, H, d), dtype=np.float32) * np.float32(d ** -0.5))
    kb = f32_to_bf16_bits(rng.standard_normal((P, n, H_kv, d), dtype=np.float32))
    vb = f32_to_bf16_bits(rng.standard_normal((P, n, H_kv, d), dtype=np.float32))
    o = torch.full((P, n, H, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = api.usp_attention(dev_bf16(qb), dev_bf16(kb), dev_bf16(vb), o, P_u=P_u, causal=True)
    torch.cuda.synchronize()
    got_o = host_f64(o).reshape(L, H, d)
    got_l = host_f64(lse).reshape(P // P_u, P_u, H // P_u, S)
    del o, lse
    q, k, v = qb.reshape(L, H, d), kb.reshape(L, H_kv, d), vb.reshape(L, H_kv, d)
    tokens = sorted({0, 1, n - 1, n, S - 1, S, L // 2, L - 1, *(int(t) for t in rng.integers(0, L, size=4))})
    for h in (0, 13, H - 1):
        g = h // (H // H_kv)
        kg, vg = bf16_bits_to_f64(k[:, g]), bf16_bits_to_f64(v[:, g])
        for t in tokens:
            ref_o, ref_l = oracle.attention_fp64(bf16_bits_to_f64(q[t, h])[None, None, None], kg[None, None, :t + 1],
                                                 vg[None, None, :t + 1])
            check_close(got_o[t, h][None, None, None], ref_o, "bf16", f"O token {t} head {h}")
            i_r, s, i_u, hl = t // S, t % S, h // (H // P_u), h % (H // P_u)
            check_close(np.array([[[got_l[i_r, i_u, hl, s]]]]), ref_l, "bf16", f"lse token {t} head {h}")

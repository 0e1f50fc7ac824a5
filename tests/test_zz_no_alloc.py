"""ra_zigzag_attention_noalloc (the zigzag ring attention whose scratch is a
file-scope device array of the library) against ra_zigzag_attention with
caller work buffers, through the C ABI: two calls in a row, the second with a
smaller input, both bit-identical to the allocating entry point and within
the bf16 bar of the fp64 oracle; sizes above the array are refused."""
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


def _case(P, c, Hq, Hkv, d, seed):
    n = 2 * c
    rng = np.random.default_rng(seed)
    bits = lambda s, sc=1.0: f32_to_bf16_bits(rng.standard_normal(s, dtype=np.float32) * np.float32(sc))
    return (bits((P, 1, Hq, n, d), d ** -0.5), bits((P, 1, Hkv, n, d)), bits((P, 1, Hkv, n, d)))


def _run_both(api, qb, kb, vb):
    P, B, Hq, n, d = qb.shape
    c = n // 2
    qd, kd, vd = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb)
    outs = []
    for r in range(P):
        o_ref = torch.full((B, Hq, n, d), float("nan"), dtype=torch.bfloat16, device="cuda")
        l_ref = torch.full((B * Hq * n,), float("nan"), dtype=torch.float32, device="cuda")
        work = (torch.empty((B, Hq, c, d), dtype=torch.float32, device="cuda"),
                torch.empty(B * Hq * c, dtype=torch.float32, device="cuda"))
        api.ra_zigzag_attention(qd[r], kd, vd, o_ref, l_ref, rank=r, work=work)
        o = torch.full_like(o_ref, float("nan"))
        lse = torch.full_like(l_ref, float("nan"))
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated()
        api.ra_zigzag_attention_noalloc(qd[r], kd, vd, o, lse, rank=r)
        torch.cuda.synchronize()
        assert torch.cuda.memory_allocated() == before
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)), f"O differs from the allocating call, rank {r}"
        assert torch.equal(lse.view(torch.int32), l_ref.view(torch.int32)), f"lse differs, rank {r}"
        outs.append((host_f64(o), host_f64(lse).reshape(B, Hq, n)))
    return outs


def _check_oracle(outs, qb, kb, vb):
    P, B, Hq, n, d = qb.shape
    kh, vh = bf16_bits_to_f64(kb), bf16_bits_to_f64(vb)
    for r, (o, l) in enumerate(outs):
        ref_o, ref_l = oracle.zigzag_attention_fp64(bf16_bits_to_f64(qb[r]), kh, vh, r)
        check_close(o, ref_o, "bf16", f"O rank {r}")
        check_close(l, ref_l, "bf16", f"lse rank {r}")


def test_noalloc_matches_allocating_entry_point(api):
    say("zigzag no-alloc: first call P=4 c=100 Hq=4 Hkv=2 d=128")
    big = _case(4, 100, 4, 2, 128, seed=3001)
    _check_oracle(_run_both(api, *big), *big)
    say("zigzag no-alloc: second, smaller call P=2 c=40 Hq=2 Hkv=1 d=64")
    small = _case(2, 40, 2, 1, 64, seed=3002)
    _check_oracle(_run_both(api, *small), *small)


def test_noalloc_refuses_above_its_scratch(api):
    """131072 rows of 129 fp32 values exceed the 64 MiB array: refused on the host."""
    say("zigzag no-alloc: size above the scratch array")
    assert api.zigzag_noalloc_max_bytes() == 64 << 20
    B, Hq, n, d = 1, 32, 8192, 128
    q = torch.zeros((B, Hq, n, d), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((1, B, Hq, n, d), dtype=torch.bfloat16, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty(B * Hq * n, dtype=torch.float32, device="cuda")
    with pytest.raises(api.SqkvError, match="scratch"):
        api.ra_zigzag_attention_noalloc(q, kv, kv, o, lse, rank=0)

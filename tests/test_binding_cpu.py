"""The Python binding checks what the C ABI cannot see: that the tensors of one
call agree in shape and dtype (a key pool with another head dim or element
type would otherwise be read past its rows).  These checks run before any
device call, so CPU tensors exercise them."""
import pytest
import torch

api = pytest.importorskip("sequence_kv_chunk_amd.api")


def _t(*shape, dtype=torch.bfloat16):
    return torch.zeros(shape, dtype=dtype)


def _ring_args(P=2, B=1, Hq=4, Hkv=2, n=64, d=128, kd=None, kdt=torch.bfloat16):
    kd = d if kd is None else kd
    q, o = _t(B, Hq, n, d), _t(B, Hq, n, d)
    kp, vp = _t(P, B, Hkv, n, kd, dtype=kdt), _t(P, B, Hkv, n, kd, dtype=kdt)
    lse = _t(B * Hq * n, dtype=torch.float32)
    return q, kp, vp, o, lse


def _raises(fn, *args, match, **kw):
    with pytest.raises(api.SqkvError, match=match) as e:
        fn(*args, **kw)
    assert e.value.status == api.SQKV_EINVAL


@pytest.mark.parametrize("fn", ["ra_ring_attention", "ra_ring_attention_packed", "ra_zigzag_attention",
                                "ra_zigzag_attention_noalloc"])
def test_ring_calls_check_the_pools(fn):
    f = getattr(api, fn)
    extra = (torch.zeros(1, dtype=torch.int64),) if fn.endswith("packed") else ()
    _raises(f, *_ring_args(kd=64), *extra, rank=0, match="shapes disagree")
    _raises(f, *_ring_args(kdt=torch.float32), *extra, rank=0, match="share a dtype")


def test_chunk_backward_checks_key_shape_and_dtypes():
    B, Hq, Hkv, n, d = 1, 4, 2, 64, 128
    q, do = _t(B, Hq, n, d), _t(B, Hq, n, d)
    lse, D = _t(B * Hq * n, dtype=torch.float32), _t(B * Hq * n, dtype=torch.float32)
    dq = _t(B, Hq, n, d, dtype=torch.float32)

    def call(kd=d, kdt=torch.bfloat16):
        k, v = _t(B, Hkv, n, kd, dtype=kdt), _t(B, Hkv, n, kd, dtype=kdt)
        dk, dv = _t(B, Hkv, n, kd, dtype=torch.float32), _t(B, Hkv, n, kd, dtype=torch.float32)
        api.ra_chunk_attention_bwd(q, k, v, do, lse, D, dq, dk, dv)

    _raises(call, kd=64, match="shapes disagree")
    _raises(call, kdt=torch.float32, match="share a dtype")


def test_ring_backward_checks_dout():
    q, kp, vp, o, lse = _ring_args()
    D = torch.zeros_like(lse)
    dq = torch.zeros(q.shape, dtype=torch.float32)
    dkp, dvp = torch.zeros(kp.shape, dtype=torch.float32), torch.zeros(vp.shape, dtype=torch.float32)
    _raises(api.ra_ring_attention_bwd, q, kp, vp, o.float(), lse, D, dq, dkp, dvp, rank=0, match="share a dtype")
    q2, kp2, vp2, _, _ = _ring_args(kd=64)
    _raises(api.ra_ring_attention_bwd, q2, kp2, vp2, o, lse, D, dq, torch.zeros(kp2.shape), torch.zeros(vp2.shape),
            rank=0, match="shapes disagree")


def test_usp_checks_work_dtype():
    P, n, H, d = 2, 64, 4, 128
    q, o = _t(P, n, H, d), _t(P, n, H, d)
    k, v = _t(P, n, 2, d), _t(P, n, 2, d)
    work = (_t(1, 2, 2 * n, H // 2, d), _t(1, 2, 2 * n, 1, d, dtype=torch.float32), _t(1, 2, 2 * n, 1, d),
            _t(1, 2, 2 * n, H // 2, d))
    _raises(api.usp_attention, q, k, v, o, P_u=2, work=work, match="bf16")

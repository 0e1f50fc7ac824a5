"""The C-ABI library loads, exports every symbol include/sqkv.h declares, and
rejects invalid arguments on the host before any HIP call (no GPU needed).

The invalid-argument cases pass fake, never-dereferenced device addresses; each
case is built so that validation must fail, which is also asserted.  They are
skipped on a machine with a visible GPU (the same cases run there against real
allocations in test_gpu_validation.py)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sqkv.h")
LIB = os.path.join(ROOT, "sequence_kv_chunk_amd", "libsqkv.so")

EINVAL, EUNSUP = 1, 2
F32, BF16 = 0, 1


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libsqkv.so is not built (run __graft_entry__.build())")
    return ctypes.CDLL(LIB)


def test_header_declares_the_api():
    names = declared_functions()
    for n in ("ra_chunk_attention", "ra_ring_attention", "ra_zigzag_attention", "ra_lse_merge",
              "ulysses_seq_to_head", "ulysses_head_to_seq", "sqkv_last_error"):
        assert n in names


def test_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} declared in sqkv.h but not exported"


def test_binding_signatures_cover_header():
    src = open(os.path.join(ROOT, "sequence_kv_chunk_amd", "api.py")).read()
    for name in declared_functions():
        assert f"_lib.{name}.argtypes" in src, f"binding lacks a signature for {name}"


def _gpu_visible():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


no_gpu = pytest.mark.skipif(_gpu_visible(), reason="fake-pointer validation only on GPU-less hosts")


class View(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("sb", ctypes.c_int64), ("sh", ctypes.c_int64), ("sn", ctypes.c_int64)]


def _setup(lib):
    V = View
    i, i64, f, vp = ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p
    lib.ra_chunk_attention.argtypes = [V, V, V, V, vp, V, vp, i, i, i, i, i, i, i, i, i, f, i, i64, i64, vp]
    lib.ra_ring_attention.argtypes = [V, V, V, i64, i64, V, vp, i, i, i, i, i, i, i, i, i, f, i, vp]
    lib.ra_zigzag_attention.argtypes = [V, V, V, i64, i64, V, vp, vp, vp, i, i, i, i, i, i, i, i, i, f, vp]
    lib.ra_lse_merge.argtypes = [V, vp, i, V, vp, i, V, vp, i, i, i, i, i, vp]
    lib.ulysses_seq_to_head.argtypes = [vp, vp, i, i64, i, i, i, i, vp]
    lib.ulysses_head_to_seq.argtypes = [vp, vp, i, i64, i, i, i, vp]
    lib.sqkv_last_error.restype = ctypes.c_char_p


GB = 1 << 30
BASE = 0            # device address the offsets below are relative to


def at(off):
    """Device address BASE + off (None stays None)."""
    return None if off is None else BASE + off


def _dense(off, H, n, d):
    return View(at(off), H * n * d, n * d, d)


def _attn_args(**kw):
    """A valid bf16 chunk-attention call on fake, disjoint addresses, overridden by kw."""
    B, Hq, Hkv, nq, nk, d = 1, 4, 2, 64, 64, 128
    a = dict(q=_dense(1 * GB, Hq, nq, d), k=_dense(2 * GB, Hkv, nk, d), v=_dense(3 * GB, Hkv, nk, d),
             o_in=View(None, 0, 0, 0), lse_in=None, o_out=_dense(4 * GB, Hq, nq, d), lse_out=at(5 * GB),
             B=B, Hq=Hq, Hkv=Hkv, n_q=nq, n_k=nk, d=d, in_dt=BF16, acc_dt=F32, out_dt=BF16, scale=0.5,
             causal=0, q_pos0=0, k_pos0=0, stream=None)
    a.update(kw)
    return a


def _call_attn(lib, a):
    return lib.ra_chunk_attention(a["q"], a["k"], a["v"], a["o_in"], a["lse_in"], a["o_out"], a["lse_out"],
                                  a["B"], a["Hq"], a["Hkv"], a["n_q"], a["n_k"], a["d"], a["in_dt"], a["acc_dt"],
                                  a["out_dt"], a["scale"], a["causal"], a["q_pos0"], a["k_pos0"], a["stream"])


ATTN_BAD = [   # (name, overrides built at call time, expected status)
    ("d=96", lambda: dict(d=96), EUNSUP),
    ("Hq%Hkv", lambda: dict(Hq=6, Hkv=4), EINVAL),
    ("scale=0", lambda: dict(scale=0.0), EINVAL),
    ("scale<0", lambda: dict(scale=-1.0), EINVAL),
    ("scale=inf", lambda: dict(scale=float("inf")), EINVAL),
    ("null q", lambda: dict(q=View(None, 0, 0, 0)), EINVAL),
    ("null lse_out", lambda: dict(lse_out=None), EINVAL),
    ("null k", lambda: dict(k=View(None, 0, 0, 0)), EINVAL),
    ("o_in without lse_in", lambda: dict(o_in=_dense(6 * GB, 4, 64, 128)), EINVAL),
    ("negative size", lambda: dict(n_q=-1), EINVAL),
    ("bad dtype", lambda: dict(in_dt=7), EUNSUP),
    ("2^32 bf16 work items", lambda: dict(n_q=1 << 30, Hq=1024), EUNSUP),
    ("fp32 rows beyond the grid", lambda: dict(n_q=1 << 30, in_dt=F32), EUNSUP),
    ("misaligned q ptr", lambda: dict(q=View(at(1 * GB + 8), 4 * 64 * 128, 64 * 128, 128)), EUNSUP),
    ("misaligned q stride", lambda: dict(q=View(at(1 * GB), 4 * 64 * 130, 64 * 130, 130)), EUNSUP),
    ("negative stride", lambda: dict(q=View(at(1 * GB), 0, -64 * 128, 128)), EINVAL),
    ("bf16 key rows overlap", lambda: dict(k=View(at(2 * GB), 2 * 64 * 128, 64 * 128, 64)), EUNSUP),
    ("bf16 value rows overlap", lambda: dict(v=View(at(3 * GB), 2 * 64 * 128, 64 * 128, 0)), EUNSUP),
    ("o_out overlaps q", lambda: dict(o_out=_dense(1 * GB + 4096, 4, 64, 128)), EINVAL),
    ("o_out rows overlap", lambda: dict(o_out=View(at(4 * GB), 4 * 64 * 128, 64 * 128, 64)), EINVAL),
    ("o_out heads alias", lambda: dict(o_out=View(at(4 * GB), 64 * 128, 0, 128)), EINVAL),
    ("lse_out overlaps k", lambda: dict(lse_out=at(2 * GB + 64)), EINVAL),
    ("o_out partially overlaps o_in", lambda: dict(o_in=_dense(6 * GB, 4, 64, 128), lse_in=at(7 * GB),
                                            o_out=_dense(6 * GB + 1024, 4, 64, 128), acc_dt=BF16), EINVAL),
    ("in-place with dtype change", lambda: dict(o_in=_dense(6 * GB, 4, 64, 128), lse_in=at(7 * GB),
                                         o_out=_dense(6 * GB, 4, 64, 128), acc_dt=F32, out_dt=BF16), EINVAL),
]


@no_gpu
@pytest.mark.parametrize("name,kw,want", ATTN_BAD, ids=[c[0] for c in ATTN_BAD])
def test_chunk_attention_rejects(lib, name, kw, want):
    check_attn_case(lib, name, kw, want)


def check_attn_case(lib, name, kw, want):
    _setup(lib)
    st = _call_attn(lib, _attn_args(**kw()))
    assert st == want, f"{name}: got {st}"
    assert lib.sqkv_last_error().decode() != ""


@no_gpu
def test_ring_rejects(lib):
    check_ring(lib)


def check_ring(lib):
    _setup(lib)
    q, k, v = _dense(1 * GB, 4, 64, 128), _dense(2 * GB, 4, 64, 128), _dense(3 * GB, 4, 64, 128)
    o, lse, none = _dense(4 * GB, 4, 64, 128), at(5 * GB), View(None, 0, 0, 0)
    cs = 4 * 64 * 128

    def call(P=4, rank=0, out_dt=BF16, causal=0, kcs=cs):
        return lib.ra_ring_attention(q, k, v, kcs, cs, o, lse, 1, 4, 4, 64, 128, P, rank, BF16, out_dt,
                                     1.0, causal, None)

    assert call(rank=4) == EINVAL
    assert call(rank=-1) == EINVAL
    assert call(P=0) == EINVAL
    assert call(kcs=cs + 3) == EUNSUP
    # the pool of 4 chunks reaches into o when o sits right after chunk 0
    assert lib.ra_ring_attention(q, k, v, cs, cs, _dense(2 * GB + 2 * cs, 4, 64, 128), lse, 1, 4, 4, 64,
                                 128, 4, 1, BF16, F32, 1.0, 0, None) == EINVAL


@no_gpu
def test_zigzag_rejects(lib):
    check_zigzag(lib)


def check_zigzag(lib):
    _setup(lib)
    q, k, v = _dense(1 * GB, 4, 64, 128), _dense(2 * GB, 4, 64, 128), _dense(3 * GB, 4, 64, 128)
    o, lse = _dense(4 * GB, 4, 64, 128), at(5 * GB)
    cs = 4 * 64 * 128

    def call(P=4, rank=0, n=64, wo=6 * GB, wl=7 * GB, kcs=cs):
        return lib.ra_zigzag_attention(q, k, v, kcs, cs, o, lse, at(wo), at(wl), 1, 4, 4, n, 128, P, rank, BF16,
                                       BF16, 1.0, None)

    assert call(rank=4) == EINVAL
    assert call(P=0) == EINVAL
    assert call(n=63) == EINVAL                  # two pieces of equal length
    assert call(wo=None) == EINVAL
    assert call(wl=None) == EINVAL
    assert call(wo=6 * GB + 4) == EUNSUP         # work_o not 16-byte aligned
    assert call(wo=4 * GB + 64) == EINVAL        # scratch inside o
    assert call(wl=5 * GB + 16) == EINVAL        # scratch inside lse
    assert call(kcs=cs + 3) == EUNSUP


@no_gpu
def test_usp_rejects(lib):
    check_usp(lib)


def check_usp(lib):
    _setup(lib)
    vp, i, i64, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float
    lib.usp_attention.argtypes = [vp] * 9 + [i, i, i64, i, i, i, f, i, vp]
    bufs = [at(g * GB) for g in range(1, 10)]

    def call(P_u=2, P_r=2, L=1024, H=4, H_kv=2, bufs=bufs, d=128):
        return lib.usp_attention(*bufs, P_u, P_r, L, H, H_kv, d, 1.0, 1, None)

    assert call(P_u=0) == EINVAL
    assert call(L=1023) == EINVAL               # not a multiple of P_u * P_r
    assert call(H=6, H_kv=2, P_u=4) == EINVAL   # H % P_u
    assert call(H=6, H_kv=3, P_u=2) == EINVAL   # H_kv and P_u: neither divides the other
    assert call(bufs=[None] + bufs[1:]) == EINVAL
    assert call(bufs=bufs[:4] + [bufs[0]] + bufs[5:]) == EINVAL   # work_q overlaps q
    assert call(d=96) == EUNSUP
    assert call(L=1 << 32) == EUNSUP                             # ring chunks of 2^31 tokens
    assert call(bufs=bufs[:5] + [at(6 * GB + 8)] + bufs[6:]) == EUNSUP   # work_k misaligned
    assert call(bufs=bufs[:8] + [at(9 * GB + 2)]) == EUNSUP              # lse misaligned


@no_gpu
def test_merge_rejects(lib):
    check_merge(lib)


def check_merge(lib):
    _setup(lib)
    a, b, o = _dense(1 * GB, 4, 8, 64), _dense(2 * GB, 4, 8, 64), _dense(3 * GB, 4, 8, 64)

    def call(d=64, oa=a, ob=b, oo=o, la=4 * GB, lb=5 * GB, lo=6 * GB, dt=F32, n=8):
        return lib.ra_lse_merge(oa, at(la), dt, ob, at(lb), dt, oo, at(lo), dt, 1, 4, n, d, None)

    assert call(d=32) == EUNSUP
    assert call(la=None) == EINVAL
    assert call(oo=_dense(1 * GB + 256, 4, 8, 64)) == EINVAL
    assert call(lo=4 * GB + 4) == EINVAL
    assert call(dt=5) == EUNSUP
    assert call(n=1 << 27, d=128) == EUNSUP      # n*d/4 = 2^32 threads in one grid row
    assert call(oo=View(at(3 * GB), 4 * 8 * 64, 0, 64)) == EINVAL   # every head writes the same rows


@no_gpu
def test_ulysses_rejects(lib):
    check_ulysses(lib)


def check_ulysses(lib):
    _setup(lib)
    s2h, h2s = lib.ulysses_seq_to_head, lib.ulysses_head_to_seq
    src, dst = at(1 * GB), at(2 * GB)
    assert s2h(src, dst, 4, 10, 8, 8, 2, 2, None) == EINVAL        # L % P
    assert s2h(src, dst, 3, 12, 8, 8, 2, 2, None) == EINVAL        # H % P
    assert s2h(src, dst, 8, 16, 4, 4, 2, 2, None) == EINVAL        # P > H
    assert s2h(src, dst, 4, 16, 8, 12, 2, 2, None) == EINVAL       # H_dst % P
    assert s2h(src, dst, 4, 16, 3, 8, 2, 2, None) == EINVAL        # H_dst % H_src
    assert s2h(src, dst, 4, 16, 8, 8, 2, 3, None) == EINVAL        # elem_bytes
    assert s2h(None, dst, 4, 16, 8, 8, 2, 2, None) == EINVAL
    assert s2h(src, src + 64, 4, 16, 8, 8, 2, 2, None) == EINVAL   # overlap
    assert s2h(src + 1, dst, 4, 16, 8, 8, 2, 2, None) == EUNSUP    # misaligned element
    assert h2s(src, dst, 4, 10, 8, 2, 2, None) == EINVAL
    assert h2s(src, dst, 8, 16, 4, 2, 2, None) == EINVAL
    assert lib.sqkv_last_error().decode() != ""


@no_gpu
def test_bwd_rejects(lib):
    check_bwd(lib)


def check_bwd(lib):
    """The backward copies q, dout, k and v tiles as rows x row stride, so a
    view whose rows overlap (row stride below d) is refused."""
    _setup(lib)
    V, i, i64, f, vp = View, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p
    lib.ra_chunk_attention_bwd.argtypes = [V, V, V, V, vp, vp, V, V, V, i, i, i, i, i, i, i, f, i, i64, i64, vp]
    H, n, d = 2, 64, 128
    views = dict(q=_dense(1 * GB, H, n, d), k=_dense(2 * GB, H, n, d), v=_dense(3 * GB, H, n, d),
                 dout=_dense(4 * GB, H, n, d), dq=_dense(6 * GB, H, n, d), dk=_dense(7 * GB, H, n, d),
                 dv=_dense(8 * GB, H, n, d))

    def call(nq=n, nk=n, **kw):
        a = dict(views, **kw)
        return lib.ra_chunk_attention_bwd(a["q"], a["k"], a["v"], a["dout"], at(5 * GB), at(5 * GB + (1 << 20)),
                                          a["dq"], a["dk"], a["dv"], 1, H, H, nq, nk, d, BF16, 1.0, 0, 0, 0, None)

    for name in ("q", "k", "v", "dout"):
        overlapping = View(at(views[name].ptr - BASE), H * n * d, n * d, 64)
        assert call(**{name: overlapping}) == EUNSUP, name
        assert b"overlap" in lib.sqkv_last_error()
    # 2^23 workgroups of either kernel
    assert call(nq=1 << 30) == EUNSUP and b"2^23" in lib.sqkv_last_error()
    assert call(nk=1 << 29) == EUNSUP and b"2^23" in lib.sqkv_last_error()
    # gradient rows that would be written twice
    assert call(dq=View(at(6 * GB), H * n * d, n * d, d // 2)) == EINVAL
    assert call(dk=View(at(7 * GB), H * n * d, 0, d)) == EINVAL        # both heads' dK in the same rows


@no_gpu
def test_ring_bwd_rejects(lib):
    check_ring_bwd(lib)


def check_ring_bwd(lib):
    """dk and dv pools whose chunks overlap would mix chunks' gradients."""
    _setup(lib)
    V, i, i64, f, vp = View, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p
    lib.ra_ring_attention_bwd.argtypes = [V, V, V, i64, i64, V, vp, vp, V, V, V, i64, i, i, i, i, i, i, i, i, f, i, vp]
    P, H, n, d = 4, 2, 64, 128
    cs = H * n * d

    def call(dkv_cs=cs, rank=1):
        return lib.ra_ring_attention_bwd(_dense(1 * GB, H, n, d), _dense(2 * GB, H, n, d), _dense(3 * GB, H, n, d),
                                         cs, cs, _dense(4 * GB, H, n, d), at(5 * GB), at(5 * GB + (1 << 20)),
                                         _dense(6 * GB, H, n, d), _dense(7 * GB, H, n, d), _dense(8 * GB, H, n, d),
                                         dkv_cs, 1, H, H, n, d, P, rank, BF16, 1.0, 1, None)

    assert call(rank=P) == EINVAL
    assert call(dkv_cs=cs // 2) == EINVAL and b"chunks" in lib.sqkv_last_error()
    assert call(dkv_cs=0) == EINVAL


@no_gpu
def test_bwd_preprocess_rejects(lib):
    check_bwd_preprocess(lib)


def check_bwd_preprocess(lib):
    _setup(lib)
    V, i, vp = View, ctypes.c_int, ctypes.c_void_p
    lib.ra_attention_bwd_preprocess.argtypes = [V, V, vp, i, i, i, i, i, vp]

    def call(H=2, n=64, d=128, D=3 * GB):
        return lib.ra_attention_bwd_preprocess(_dense(1 * GB, H, n, d), _dense(2 * GB, H, n, d), at(D), 1, H, n, d,
                                               BF16, None)

    assert call(d=96) == EUNSUP
    assert call(D=None) == EINVAL
    assert call(D=1 * GB + 64) == EINVAL                    # D inside o
    assert call(H=16, n=1 << 24) == EUNSUP                 # 2^28 rows of 16 threads


@no_gpu
def test_empty_sizes_are_noops(lib):
    check_empty(lib)


def check_empty(lib):
    _setup(lib)
    # nothing to do: OK without touching memory
    assert _call_attn(lib, _attn_args(n_q=0)) == 0
    assert lib.ulysses_seq_to_head(at(1 * GB), at(2 * GB), 4, 0, 8, 8, 2, 2, None) == 0
    assert lib.sqkv_last_error().decode() == ""


@no_gpu
def test_zigzag_noalloc_refuses_on_the_host(lib):
    """The no-allocation zigzag variant validates like ra_zigzag_attention and
    refuses partials larger than its scratch array before any HIP call."""
    _setup(lib)
    i, i64, f, vp = ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p
    V = View
    lib.ra_zigzag_attention_noalloc.argtypes = [V, V, V, i64, i64, V, vp, i, i, i, i, i, i, i, i, i, f, vp]
    lib.ra_zigzag_attention_noalloc_max_bytes.restype = ctypes.c_size_t
    assert lib.ra_zigzag_attention_noalloc_max_bytes() == 64 << 20
    H, n, d = 32, 8192, 128          # 131072 rows of 129 fp32 values: above 64 MiB
    q, k, v = _dense(1 * GB, H, n, d), _dense(2 * GB, H, n, d), _dense(3 * GB, H, n, d)
    o, lse = _dense(4 * GB, H, n, d), at(5 * GB)

    def call(n=n, rank=0):
        return lib.ra_zigzag_attention_noalloc(q, k, v, 0, 0, o, lse, 1, H, H, n, d, 1, rank, BF16, BF16, 1.0,
                                               None)

    assert call() == EUNSUP and b"scratch" in lib.sqkv_last_error()
    assert call(n=n - 1) == EINVAL           # odd shard: refused before the size check
    assert call(rank=1) == EINVAL

"""Thin ctypes binding of libsqkv (include/sqkv.h) for torch tensors.

Argument marshalling only: every function passes device pointers, element
strides, sizes and the current HIP stream of the tensors' device to the C ABI
and raises ``SqkvError`` with the library's message on a non-OK status.  All
computation happens in the HIP kernels; there is no fallback path.  Importing
this module loads ``libsqkv.so`` and fails loudly if it has not been built.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("SQKV_LIB", os.path.join(_HERE, "libsqkv.so"))

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"libsqkv.so not found at {LIB_PATH}; build it with `python -m sequence_kv_chunk_amd.build` "
        "(or __graft_entry__.build()) -- there is no non-HIP fallback")

_lib = ctypes.CDLL(LIB_PATH)

SQKV_OK, SQKV_EINVAL, SQKV_EUNSUPPORTED, SQKV_EHIP = 0, 1, 2, 3
SQKV_F32, SQKV_BF16 = 0, 1
STATUS_NAMES = {0: "SQKV_OK", 1: "SQKV_EINVAL", 2: "SQKV_EUNSUPPORTED", 3: "SQKV_EHIP"}


class SqkvView(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("sb", ctypes.c_int64), ("sh", ctypes.c_int64),
                ("sn", ctypes.c_int64)]


class SqkvError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_c_int, _c_i64, _c_f, _vp = ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p
_V = SqkvView

_lib.sqkv_last_error.restype = ctypes.c_char_p
_lib.sqkv_last_error.argtypes = []
_lib.ra_chunk_attention.restype = _c_int
_lib.ra_chunk_attention.argtypes = [_V, _V, _V, _V, _vp, _V, _vp, _c_int, _c_int, _c_int, _c_int, _c_int,
                                    _c_int, _c_int, _c_int, _c_int, _c_f, _c_int, _c_i64, _c_i64, _vp]
_lib.ra_ring_attention.restype = _c_int
_lib.ra_ring_attention.argtypes = [_V, _V, _V, _c_i64, _c_i64, _V, _vp, _c_int, _c_int, _c_int, _c_int,
                                   _c_int, _c_int, _c_int, _c_int, _c_int, _c_f, _c_int, _vp]
_lib.ra_zigzag_attention.restype = _c_int
_lib.ra_zigzag_attention.argtypes = [_V, _V, _V, _c_i64, _c_i64, _V, _vp, _vp, _vp, _c_int, _c_int, _c_int,
                                     _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_f, _vp]
_lib.ra_zigzag_attention_noalloc.restype = _c_int
_lib.ra_zigzag_attention_noalloc.argtypes = [_V, _V, _V, _c_i64, _c_i64, _V, _vp, _c_int, _c_int, _c_int, _c_int,
                                             _c_int, _c_int, _c_int, _c_int, _c_int, _c_f, _vp]
_lib.ra_zigzag_attention_noalloc_max_bytes.restype = ctypes.c_size_t
_lib.ra_zigzag_attention_noalloc_max_bytes.argtypes = []
_lib.ra_attention_bwd_preprocess.restype = _c_int
_lib.ra_attention_bwd_preprocess.argtypes = [_V, _V, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _vp]
_lib.ra_chunk_attention_bwd.restype = _c_int
_lib.ra_chunk_attention_bwd.argtypes = [_V, _V, _V, _V, _vp, _vp, _V, _V, _V, _c_int, _c_int, _c_int, _c_int,
                                        _c_int, _c_int, _c_int, _c_f, _c_int, _c_i64, _c_i64, _vp]
_lib.ra_ring_attention_bwd.restype = _c_int
_lib.ra_ring_attention_bwd.argtypes = [_V, _V, _V, _c_i64, _c_i64, _V, _vp, _vp, _V, _V, _V, _c_i64, _c_int,
                                       _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_f, _c_int, _vp]
_lib.usp_attention.restype = _c_int
_lib.usp_attention.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_i64, _c_int, _c_int,
                               _c_int, _c_f, _c_int, _vp]
_lib.ra_ring_attention_packed.restype = _c_int
_lib.ra_ring_attention_packed.argtypes = [_V, _V, _V, _c_i64, _c_i64, _V, _vp, _vp, _c_int, _c_int, _c_int, _c_int,
                                          _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_f, _vp]
_lib.ra_lse_merge.restype = _c_int
_lib.ra_lse_merge.argtypes = [_V, _vp, _c_int, _V, _vp, _c_int, _V, _vp, _c_int, _c_int, _c_int, _c_int,
                              _c_int, _vp]
_lib.ulysses_seq_to_head.restype = _c_int
_lib.ulysses_seq_to_head.argtypes = [_vp, _vp, _c_int, _c_i64, _c_int, _c_int, _c_int, _c_int, _vp]
_lib.ulysses_head_to_seq.restype = _c_int
_lib.ulysses_head_to_seq.argtypes = [_vp, _vp, _c_int, _c_i64, _c_int, _c_int, _c_int, _vp]

EXPORTED = ("ra_chunk_attention", "ra_ring_attention", "ra_ring_attention_packed", "ra_zigzag_attention",
            "ra_zigzag_attention_noalloc", "ra_zigzag_attention_noalloc_max_bytes", "ra_lse_merge",
            "ra_attention_bwd_preprocess", "ra_chunk_attention_bwd", "ra_ring_attention_bwd",
            "ulysses_seq_to_head", "ulysses_head_to_seq", "usp_attention", "sqkv_last_error")


def _check(status: int):
    if status != SQKV_OK:
        raise SqkvError(status, _lib.sqkv_last_error().decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return SQKV_F32
    if t.dtype == torch.bfloat16:
        return SQKV_BF16
    raise SqkvError(SQKV_EUNSUPPORTED, f"dtype {t.dtype} (need float32 or bfloat16)")


def _bhnd(t: torch.Tensor) -> torch.Tensor:
    """[B, H, n, d] as is; a [S, H, d] Ulysses share becomes the view [1, H, S, d]."""
    if t.dim() == 3:
        return t.unsqueeze(0).transpose(1, 2)
    if t.dim() != 4:
        raise SqkvError(SQKV_EINVAL, f"expected a [B, H, n, d] or [S, H, d] tensor, got {tuple(t.shape)}")
    return t


def _view(t: torch.Tensor | None) -> SqkvView:
    if t is None:
        return SqkvView(None, 0, 0, 0)
    if t.stride(-1) != 1:
        raise SqkvError(SQKV_EINVAL, "innermost (d) stride must be 1")
    # a single row's stride is never used: pass one that cannot make rows overlap
    sn = t.stride(2) if t.shape[2] != 1 else max(t.stride(2), t.shape[3])
    return SqkvView(t.data_ptr(), t.stride(0), t.stride(1), sn)


def _stream(t: torch.Tensor) -> int:
    if not t.is_cuda:
        raise SqkvError(SQKV_EINVAL, "tensors must live on a GPU")
    return torch.cuda.current_stream(t.device).cuda_stream


def _same_device(*ts):
    devs = {t.device for t in ts if t is not None}
    if len(devs) != 1:
        raise SqkvError(SQKV_EINVAL, f"tensors on different devices: {devs}")


def _same_dtype(what: str, *ts):
    if len({t.dtype for t in ts}) != 1:
        raise SqkvError(SQKV_EINVAL, f"{what} must share a dtype")


def _ring_shapes(q, k_pool, v_pool, o):
    """(P, B, Hq, Hkv, n, d) of a ring call, after checking that q, o
    ([B, Hq, n, d]) and the pools ([P, B, Hkv, n, d]) agree."""
    if k_pool.dim() != 5 or v_pool.shape != k_pool.shape:
        raise SqkvError(SQKV_EINVAL, "k_pool, v_pool must be [P, B, Hkv, n, d]")
    if q.dim() != 4:
        raise SqkvError(SQKV_EINVAL, f"q must be [B, Hq, n, d], got {tuple(q.shape)}")
    P, Bk, Hkv, nk, dk = k_pool.shape
    B, Hq, n, d = q.shape
    if tuple(o.shape) != (B, Hq, n, d) or (Bk, nk, dk) != (B, n, d):
        raise SqkvError(SQKV_EINVAL, "shapes disagree")
    _same_dtype("q, k_pool and v_pool", q, k_pool, v_pool)
    return P, B, Hq, Hkv, n, d


def _lse_ptr(t: torch.Tensor | None, rows: int):
    if t is None:
        return None
    if t.dtype != torch.float32 or not t.is_contiguous() or t.numel() != rows:
        raise SqkvError(SQKV_EINVAL, f"lse must be a dense float32 tensor of {rows} elements")
    return t.data_ptr()


def ra_chunk_attention(q, k, v, o_out, lse_out, *, o_in=None, lse_in=None, scale: float = 1.0,
                       causal: bool = False, q_pos0: int = 0, k_pos0: int = 0):
    """One ring step: merge attention of ``q`` over chunk (k, v) into (o_in, lse_in)
    (or write the chunk's own partial when o_in is None) as (o_out, lse_out)."""
    q4, k4, v4, oo4 = _bhnd(q), _bhnd(k), _bhnd(v), _bhnd(o_out)
    oi4 = _bhnd(o_in) if o_in is not None else None
    _same_device(q4, k4, v4, oo4, oi4, lse_out, lse_in)
    B, Hq, n_q, d = q4.shape
    Hkv, n_k = k4.shape[1], k4.shape[2]
    if k4.shape != v4.shape or tuple(oo4.shape) != (B, Hq, n_q, d) or k4.shape[0] != B or k4.shape[3] != d:
        raise SqkvError(SQKV_EINVAL, "q/k/v/o shapes disagree")
    if oi4 is not None and tuple(oi4.shape) != (B, Hq, n_q, d):
        raise SqkvError(SQKV_EINVAL, "o_in shape disagrees")
    if q4.dtype != k4.dtype or q4.dtype != v4.dtype:
        raise SqkvError(SQKV_EINVAL, "q, k, v must share a dtype")
    rows = B * Hq * n_q
    acc_dt = _dtype_code(oi4) if oi4 is not None else SQKV_F32
    with torch.cuda.device(q4.device):
        st = _lib.ra_chunk_attention(_view(q4), _view(k4), _view(v4), _view(oi4), _lse_ptr(lse_in, rows),
                                     _view(oo4), _lse_ptr(lse_out, rows), B, Hq, Hkv, n_q, n_k, d,
                                     _dtype_code(q4), acc_dt, _dtype_code(oo4), float(scale), int(bool(causal)),
                                     int(q_pos0), int(k_pos0), _stream(q4))
    _check(st)


def ra_ring_attention(q, k_pool, v_pool, o, lse, *, rank: int, scale: float = 1.0, causal: bool = False):
    """Ring attention of query chunk ``q`` ([B, Hq, n, d]) of virtual rank ``rank``
    over the P resident chunks of ``k_pool``/``v_pool`` ([P, B, Hkv, n, d])."""
    _same_device(q, k_pool, v_pool, o, lse)
    P, B, Hq, Hkv, n, d = _ring_shapes(q, k_pool, v_pool, o)
    with torch.cuda.device(q.device):
        st = _lib.ra_ring_attention(_view(q), _view(k_pool[0]), _view(v_pool[0]), k_pool.stride(0),
                                    v_pool.stride(0), _view(o), _lse_ptr(lse, B * Hq * n),
                                    B, Hq, k_pool.shape[2], n, d, P, int(rank), _dtype_code(q),
                                    _dtype_code(o), float(scale), int(bool(causal)), _stream(q))
    _check(st)


def ra_ring_attention_packed(q, k_pool, v_pool, o, lse, seg_starts, *, rank: int, scale: float = 1.0):
    """Causal ring attention of virtual rank ``rank`` over a packed sequence:
    ``seg_starts`` (int64 device tensor) holds the samples' start positions in
    the whole sequence; a query sees only keys of its own sample."""
    _same_device(q, k_pool, v_pool, o, lse, seg_starts)
    if seg_starts.dtype != torch.int64 or seg_starts.dim() != 1 or not seg_starts.is_contiguous():
        raise SqkvError(SQKV_EINVAL, "seg_starts must be a contiguous 1-D int64 tensor")
    P, B, Hq, Hkv, n, d = _ring_shapes(q, k_pool, v_pool, o)
    with torch.cuda.device(q.device):
        st = _lib.ra_ring_attention_packed(_view(q), _view(k_pool[0]), _view(v_pool[0]), k_pool.stride(0),
                                           v_pool.stride(0), _view(o), _lse_ptr(lse, B * Hq * n), seg_starts.data_ptr(),
                                           seg_starts.numel(), B, Hq, k_pool.shape[2], n, d, P, int(rank),
                                           _dtype_code(q), _dtype_code(o), float(scale), _stream(q))
    _check(st)


def ra_zigzag_attention(q, k_pool, v_pool, o, lse, *, rank: int, scale: float = 1.0, work=None):
    """Causal ring attention of virtual rank ``rank`` under the zigzag split:
    ``q`` ([B, Hq, n, d]) holds the rank's pieces ``rank`` and ``2P-1-rank``
    of the 2P-piece sequence, ``k_pool``/``v_pool`` ([P, B, Hkv, n, d]) every
    rank's shard in the same layout.  ``work`` = (work_o fp32 [B, Hq, n/2, d],
    work_lse fp32 [B*Hq*n/2]) scratch; allocated here when not given."""
    _same_device(q, k_pool, v_pool, o, lse)
    P, B, Hq, Hkv, n, d = _ring_shapes(q, k_pool, v_pool, o)
    if work is None:
        work = (torch.empty((B, Hq, n // 2, d), dtype=torch.float32, device=q.device),
                torch.empty(B * Hq * (n // 2), dtype=torch.float32, device=q.device))
    wo, wl = work
    _same_device(q, wo, wl)
    if wo.dtype != torch.float32 or wl.dtype != torch.float32 or not wo.is_contiguous() or not wl.is_contiguous() \
            or wo.numel() != B * Hq * (n // 2) * d or wl.numel() != B * Hq * (n // 2):
        raise SqkvError(SQKV_EINVAL, "work must be contiguous fp32 [B, Hq, n/2, d] and [B*Hq*n/2]")
    with torch.cuda.device(q.device):
        st = _lib.ra_zigzag_attention(_view(q), _view(k_pool[0]), _view(v_pool[0]), k_pool.stride(0),
                                      v_pool.stride(0), _view(o), _lse_ptr(lse, B * Hq * n), wo.data_ptr(),
                                      wl.data_ptr(), B, Hq, k_pool.shape[2], n, d, P, int(rank), _dtype_code(q),
                                      _dtype_code(o), float(scale), _stream(q))
    _check(st)


def ra_zigzag_attention_noalloc(q, k_pool, v_pool, o, lse, *, rank: int, scale: float = 1.0):
    """ra_zigzag_attention with the late piece's partial in the library's own
    per-GPU scratch array instead of caller work buffers: allocates nothing,
    for callers that cannot.  Calls that overlap on one GPU race on that
    scratch.  B*Hq*n/2 rows must fit zigzag_noalloc_max_bytes()."""
    _same_device(q, k_pool, v_pool, o, lse)
    P, B, Hq, Hkv, n, d = _ring_shapes(q, k_pool, v_pool, o)
    with torch.cuda.device(q.device):
        st = _lib.ra_zigzag_attention_noalloc(_view(q), _view(k_pool[0]), _view(v_pool[0]), k_pool.stride(0),
                                              v_pool.stride(0), _view(o), _lse_ptr(lse, B * Hq * n), B, Hq,
                                              k_pool.shape[2], n, d, P, int(rank), _dtype_code(q), _dtype_code(o),
                                              float(scale), _stream(q))
    _check(st)


def zigzag_noalloc_max_bytes() -> int:
    """Size of the scratch array ra_zigzag_attention_noalloc works in."""
    return int(_lib.ra_zigzag_attention_noalloc_max_bytes())


def ra_attention_bwd_preprocess(o, dout, D):
    """D = rowsum(dout * o) over [B, H, n, d] tensors (or [S, H, d] shares)."""
    o4, d4 = _bhnd(o), _bhnd(dout)
    _same_device(o4, d4, D)
    B, H, n, d = o4.shape
    if d4.shape != o4.shape or d4.dtype != o4.dtype:
        raise SqkvError(SQKV_EINVAL, "o and dout must agree in shape and dtype")
    with torch.cuda.device(o4.device):
        st = _lib.ra_attention_bwd_preprocess(_view(o4), _view(d4), _lse_ptr(D, B * H * n), B, H, n, d,
                                              _dtype_code(o4), _stream(o4))
    _check(st)


def _f32(*ts):
    for t in ts:
        if t.dtype != torch.float32:
            raise SqkvError(SQKV_EINVAL, "gradient buffers must be float32")


def ra_chunk_attention_bwd(q, k, v, dout, lse, D, dq, dk, dv, *, scale: float = 1.0, causal: bool = False,
                           q_pos0: int = 0, k_pos0: int = 0):
    """Adds one chunk pair's share of (dQ, dK, dV) into the float32 dq, dk, dv."""
    q4, k4, v4, o4 = _bhnd(q), _bhnd(k), _bhnd(v), _bhnd(dout)
    g4, gk4, gv4 = _bhnd(dq), _bhnd(dk), _bhnd(dv)
    _same_device(q4, k4, v4, o4, lse, D, g4, gk4, gv4)
    _f32(g4, gk4, gv4)
    B, Hq, n_q, d = q4.shape
    Hkv, n_k = k4.shape[1], k4.shape[2]
    if o4.shape != q4.shape or g4.shape != q4.shape or v4.shape != k4.shape or gk4.shape != k4.shape \
            or gv4.shape != k4.shape or k4.shape[0] != B or k4.shape[3] != d:
        raise SqkvError(SQKV_EINVAL, "shapes disagree")
    _same_dtype("q, k, v and dout", q4, k4, v4, o4)
    rows = B * Hq * n_q
    with torch.cuda.device(q4.device):
        st = _lib.ra_chunk_attention_bwd(_view(q4), _view(k4), _view(v4), _view(o4), _lse_ptr(lse, rows),
                                         _lse_ptr(D, rows), _view(g4), _view(gk4), _view(gv4), B, Hq, Hkv, n_q,
                                         n_k, d, _dtype_code(q4), float(scale), int(bool(causal)), int(q_pos0),
                                         int(k_pos0), _stream(q4))
    _check(st)


def ra_ring_attention_bwd(q, k_pool, v_pool, dout, lse, D, dq, dk_pool, dv_pool, *, rank: int,
                          scale: float = 1.0, causal: bool = False):
    """Backward of ra_ring_attention for virtual rank ``rank``: dq [B, Hq, n, d]
    receives the rank's dQ, dk_pool/dv_pool ([P, B, Hkv, n, d] float32) the
    rank's share of every chunk's dK, dV (all accumulated)."""
    if k_pool.dim() != 5 or v_pool.shape != k_pool.shape or dk_pool.shape != k_pool.shape \
            or dv_pool.shape != k_pool.shape:
        raise SqkvError(SQKV_EINVAL, "pools must be [P, B, Hkv, n, d]")
    _same_device(q, k_pool, v_pool, dout, lse, D, dq, dk_pool, dv_pool)
    _f32(dq, dk_pool, dv_pool)
    if dk_pool.stride(0) != dv_pool.stride(0):
        raise SqkvError(SQKV_EINVAL, "dk_pool and dv_pool must share a chunk stride")
    P, B, Hq, Hkv, n, d = _ring_shapes(q, k_pool, v_pool, dout)
    if tuple(dq.shape) != (B, Hq, n, d):
        raise SqkvError(SQKV_EINVAL, "shapes disagree")
    _same_dtype("q and dout", q, dout)
    rows = B * Hq * n
    with torch.cuda.device(q.device):
        st = _lib.ra_ring_attention_bwd(_view(q), _view(k_pool[0]), _view(v_pool[0]), k_pool.stride(0),
                                        v_pool.stride(0), _view(dout), _lse_ptr(lse, rows), _lse_ptr(D, rows),
                                        _view(dq), _view(dk_pool[0]), _view(dv_pool[0]), dk_pool.stride(0), B, Hq,
                                        k_pool.shape[2], n, d, P, int(rank), _dtype_code(q), float(scale),
                                        int(bool(causal)), _stream(q))
    _check(st)


def ra_lse_merge(o_a, lse_a, o_b, lse_b, o_out, lse_out):
    """(o_out, lse_out) = merge((o_a, lse_a), (o_b, lse_b)) over [B, H, n, d] tensors."""
    a4, b4, o4 = _bhnd(o_a), _bhnd(o_b), _bhnd(o_out)
    _same_device(a4, b4, o4, lse_a, lse_b, lse_out)
    B, H, n, d = a4.shape
    if b4.shape != a4.shape or o4.shape != a4.shape:
        raise SqkvError(SQKV_EINVAL, "shapes disagree")
    rows = B * H * n
    with torch.cuda.device(a4.device):
        st = _lib.ra_lse_merge(_view(a4), _lse_ptr(lse_a, rows), _dtype_code(a4), _view(b4), _lse_ptr(lse_b, rows),
                               _dtype_code(b4), _view(o4), _lse_ptr(lse_out, rows), _dtype_code(o4), B, H, n, d,
                               _stream(a4))
    _check(st)


def _dense(t: torch.Tensor, name: str):
    if not t.is_contiguous():
        raise SqkvError(SQKV_EINVAL, f"{name} must be contiguous")


def ulysses_seq_to_head(src, dst, *, H_dst: int | None = None):
    """src [P, L/P, H_src, d] -> dst [P, L, H_dst/P, d] (H_dst defaults to H_src)."""
    _dense(src, "src"); _dense(dst, "dst")
    _same_device(src, dst)
    P, n, H_src, d = src.shape
    H_dst = H_src if H_dst is None else int(H_dst)
    if dst.dtype != src.dtype or tuple(dst.shape) != (P, P * n, H_dst // P, d):
        raise SqkvError(SQKV_EINVAL, f"dst must be {src.dtype} [{P}, {P * n}, {H_dst // P}, {d}]")
    with torch.cuda.device(src.device):
        st = _lib.ulysses_seq_to_head(src.data_ptr(), dst.data_ptr(), P, P * n, H_src, H_dst, d,
                                      src.element_size(), _stream(src))
    _check(st)


def ulysses_head_to_seq(src, dst):
    """src [P, L, H/P, d] -> dst [P, L/P, H, d]."""
    _dense(src, "src"); _dense(dst, "dst")
    _same_device(src, dst)
    P, L, Hl, d = src.shape
    if dst.dtype != src.dtype or tuple(dst.shape) != (P, L // P, Hl * P, d):
        raise SqkvError(SQKV_EINVAL, f"dst must be {src.dtype} [{P}, {L // P}, {Hl * P}, {d}]")
    with torch.cuda.device(src.device):
        st = _lib.ulysses_head_to_seq(src.data_ptr(), dst.data_ptr(), P, L, Hl * P, d, src.element_size(),
                                      _stream(src))
    _check(st)


def usp_attention(q, k, v, o, *, P_u: int, scale: float = 1.0, causal: bool = False, work=None, lse=None):
    """Ulysses inside groups of P_u virtual ranks, ring attention across the
    P_r = P / P_u groups.  q, o: [P, L/P, H, d] bf16; k, v: [P, L/P, H_kv, d]
    bf16 (sequence layout).  ``work`` = (work_q, work_k, work_v, work_o)
    scratch and ``lse`` ([P_r, P_u, H/P_u, L/P_r] float32) are allocated here
    when not given.  Returns lse."""
    for t in (q, k, v, o):
        _dense(t, "q/k/v/o")
    _same_device(q, k, v, o)
    P, n, H, d = q.shape
    H_kv = k.shape[2]
    if tuple(o.shape) != tuple(q.shape) or tuple(v.shape) != tuple(k.shape) or k.shape[:2] != q.shape[:2] \
            or q.dtype != torch.bfloat16 or k.dtype != torch.bfloat16 or v.dtype != torch.bfloat16 \
            or o.dtype != torch.bfloat16:
        raise SqkvError(SQKV_EINVAL, "q, o [P, L/P, H, d] and k, v [P, L/P, H_kv, d], all bf16")
    P_u = int(P_u)
    if P_u < 1 or P % P_u or H % P_u:
        raise SqkvError(SQKV_EINVAL, "P_u must divide P and H")
    P_r = P // P_u
    L = P * n
    S = L // P_r
    Hk = max(H_kv, P_u) // P_u
    if work is None:
        work = (torch.empty((P_r, P_u, S, H // P_u, d), dtype=torch.bfloat16, device=q.device),
                torch.empty((P_r, P_u, S, Hk, d), dtype=torch.bfloat16, device=q.device),
                torch.empty((P_r, P_u, S, Hk, d), dtype=torch.bfloat16, device=q.device),
                torch.empty((P_r, P_u, S, H // P_u, d), dtype=torch.bfloat16, device=q.device))
    if lse is None:
        lse = torch.empty((P_r, P_u, H // P_u, S), dtype=torch.float32, device=q.device)
    wq, wk, wv, wo = work
    _same_device(q, wq, wk, wv, wo, lse)
    for t in (wq, wk, wv, wo, lse):
        _dense(t, "work/lse")
    if any(t.dtype != torch.bfloat16 for t in (wq, wk, wv, wo)):
        raise SqkvError(SQKV_EINVAL, "work buffers must be bf16")
    if wq.numel() != q.numel() or wo.numel() != q.numel() or wk.numel() != P_r * P_u * S * Hk * d \
            or wv.numel() != wk.numel() or lse.numel() != P_r * P_u * (H // P_u) * S or lse.dtype != torch.float32:
        raise SqkvError(SQKV_EINVAL, "work buffers or lse have the wrong size")
    with torch.cuda.device(q.device):
        st = _lib.usp_attention(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), wq.data_ptr(),
                                wk.data_ptr(), wv.data_ptr(), wo.data_ptr(), lse.data_ptr(), P_u, P_r, L, H, H_kv,
                                d, float(scale), int(bool(causal)), _stream(q))
    _check(st)
    return lse

"""Ulysses layout kernels against the oracle's index copy: bit-exact."""
import numpy as np
import pytest

import oracle
from sequence_kv_chunk_amd.synth import (ULYSSES_WORKLOADS, tag_pattern_u16, tag_pattern_u32,
                                         ulysses_input)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from gpu_util import host_bits, say  # noqa: E402


@pytest.fixture(scope="module")
def api():
    from sequence_kv_chunk_amd import api
    return api


def _dev(bits):
    dt = {np.dtype(np.uint8): torch.uint8, np.dtype(np.uint16): torch.int16,
          np.dtype(np.uint32): torch.int32, np.dtype(np.uint64): torch.int64}[bits.dtype]
    view = {np.dtype(np.uint16): np.int16, np.dtype(np.uint32): np.int32, np.dtype(np.uint64): np.int64,
            np.dtype(np.uint8): np.uint8}[bits.dtype]
    return torch.from_numpy(np.ascontiguousarray(bits).view(view)).to("cuda").view(dt)


CASES = [
    # P, n, H_src, H_dst, d, dtype
    (1, 5, 3, 3, 4, np.uint16),
    (2, 3, 2, 2, 4, np.uint16),
    (2, 7, 4, 4, 3, np.uint16),      # 2-byte run granularity
    (4, 5, 8, 8, 16, np.uint16),
    (4, 33, 8, 8, 64, np.uint16),
    (8, 16, 32, 32, 128, np.uint16),  # 1 KiB runs, the 128k layout in miniature
    (8, 9, 16, 16, 128, np.uint16),
    (3, 4, 6, 6, 5, np.uint32),
    (4, 6, 4, 4, 2, np.uint8),
    (2, 5, 2, 2, 3, np.uint64),
    # GQA replication: H_dst = max(H_kv, P)
    (8, 6, 2, 8, 8, np.uint16),
    (8, 4, 1, 8, 128, np.uint16),
    (4, 5, 2, 4, 64, np.uint16),
    (2, 3, 1, 4, 4, np.uint32),
    (8, 16, 8, 8, 128, np.uint16),   # H_kv = P: no copies
]


def _src(P, n, H, d, dt):
    if dt == np.uint16:
        return tag_pattern_u16((P, n, H, d), seed=P * 100 + n)
    if dt == np.uint32:
        return tag_pattern_u32((P, n, H, d))
    rng = np.random.default_rng(P + n)
    return rng.integers(0, np.iinfo(dt).max, size=(P, n, H, d), dtype=dt, endpoint=True)


@pytest.mark.parametrize("P,n,Hs,Hd,d,dt", CASES)
def test_seq_to_head_bit_exact(api, P, n, Hs, Hd, d, dt):
    say(f"ulysses seq->head P={P} n={n} H={Hs}->{Hd} d={d} {np.dtype(dt).name}")
    src = _src(P, n, Hs, d, dt)
    want = oracle.seq_to_head_naive(src, P, Hd)
    s = _dev(src)
    out = torch.empty((P, P * n, Hd // P, d), dtype=s.dtype, device="cuda")
    out.fill_(-1)
    api.ulysses_seq_to_head(s, out, H_dst=Hd)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(out), want)
    if Hs == Hd:
        back = torch.empty_like(s).fill_(-1)
        api.ulysses_head_to_seq(out, back)
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(back), src), "round trip"
        assert np.array_equal(host_bits(back), oracle.head_to_seq_naive(want, P))


def test_head_to_seq_matches_oracle_on_fresh_input(api):
    P, L, Hl, d = 4, 24, 3, 8
    src = tag_pattern_u16((P, L, Hl, d), seed=7)
    want = oracle.head_to_seq_naive(src, P)
    out = torch.empty((P, L // P, Hl * P, d), dtype=torch.int16, device="cuda")
    api.ulysses_head_to_seq(_dev(src), out)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(out), want)


def test_bf16_tensors_move_bits(api):
    # special bf16 patterns (NaN payloads, -0, subnormals) through a bfloat16 tensor
    P, n, H, d = 4, 8, 8, 16
    src = tag_pattern_u16((P, n, H, d), seed=3)
    s = _dev(src).view(torch.bfloat16)
    out = torch.empty((P, P * n, H // P, d), dtype=torch.bfloat16, device="cuda")
    api.ulysses_seq_to_head(s, out)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(out), oracle.seq_to_head_naive(src, P))


@pytest.mark.slow
def test_ulysses_131k_full_size(api):
    w = ULYSSES_WORKLOADS["ulysses_131k_32h"]
    say(f"ulysses full size P={w.P} L={w.L} H={w.H} d={w.d}")
    src = ulysses_input(w)
    want = oracle.seq_to_head_naive(src, w.P)
    s = _dev(src).view(torch.bfloat16)
    mid = torch.empty((w.P, w.L, w.H // w.P, w.d), dtype=torch.bfloat16, device="cuda")
    api.ulysses_seq_to_head(s, mid)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(mid), want)
    back = torch.empty_like(s)
    api.ulysses_head_to_seq(mid, back)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(back), src)
    # GQA share at the same length: 8 KV heads over P=8 ranks (one head each)
    kv = src[:, :, :8, :].copy()
    kd = _dev(kv).view(torch.bfloat16)
    kout = torch.empty((w.P, w.L, 1, w.d), dtype=torch.bfloat16, device="cuda")
    api.ulysses_seq_to_head(kd, kout, H_dst=8)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(kout), oracle.seq_to_head_naive(kv, w.P, 8))

"""Helpers for the GPU parity tests: moving seeded bit patterns to and from the
device and comparing against the oracle at the stated tolerances."""
from __future__ import annotations

import sys

import numpy as np
import torch

from sequence_kv_chunk_amd.synth import bf16_bits_to_f64

# Tolerances (fixed by the method's acceptance bar):
#   fp32 attention : normwise relative error <= 1e-5 (max|err| / max|ref| per tensor)
#   bf16 attention : max-abs error <= 2e-2 against float64, fp32 accumulation
FP32_REL_TOL = 1e-5
BF16_ABS_TOL = 2e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_bf16(bits: np.ndarray, device="cuda") -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to(device)


def dev_f32(x: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)


def host_bits(t: torch.Tensor) -> np.ndarray:
    """Raw element bits of a device tensor (uint16 for 2-byte, uint32 for 4-byte...)."""
    t = t.detach().contiguous().cpu()
    u = {1: torch.uint8, 2: torch.int16, 4: torch.int32, 8: torch.int64}[t.element_size()]
    n = {1: np.uint8, 2: np.uint16, 4: np.uint32, 8: np.uint64}[t.element_size()]
    return t.view(u).numpy().view(n)


def host_f64(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return bf16_bits_to_f64(host_bits(t))
    return t.to(torch.float64).numpy()


def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits_to_f64(x) if dtype == "bf16" else np.asarray(x, dtype=np.float64)


def check_close(got: np.ndarray, ref: np.ndarray, dtype: str, what: str):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, f"{what}: shape {got.shape} vs {ref.shape}"
    ninf_r, ninf_g = np.isneginf(ref), np.isneginf(got)
    assert np.array_equal(ninf_r, ninf_g), f"{what}: -inf pattern differs ({ninf_r.sum()} vs {ninf_g.sum()})"
    fin = ~ninf_r
    assert np.isfinite(got[fin]).all(), f"{what}: non-finite values"
    if not fin.any():
        return 0.0
    err = np.abs(got[fin] - ref[fin])
    if dtype == "f32":
        scale = max(np.max(np.abs(ref[fin])), 1e-30)
        rel = float(np.max(err) / scale)
        assert rel <= FP32_REL_TOL, f"{what}: normwise rel err {rel:.3e} > {FP32_REL_TOL}"
        return rel
    mx = float(np.max(err))
    assert mx <= BF16_ABS_TOL, f"{what}: max abs err {mx:.3e} > {BF16_ABS_TOL}"
    return mx

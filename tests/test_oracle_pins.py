"""The CPU oracle against its pins (no GPU)."""
import pytest

import oracle
import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle)


def test_workload_flop_counts():
    """The workloads' algorithmic FLOP counts (bench.py's numerators) equal the
    visible (query, key) pairs counted from positions, times 4*d."""
    import numpy as np
    import oracle
    from sequence_kv_chunk_amd.synth import WORKLOADS
    for name, w in WORKLOADS.items():
        pairs = 0
        if w.layout == "shd":
            pairs = oracle.unmasked_pairs(w.L, w.L, w.causal)
        elif w.layout == "zigzag":
            c = w.n // 2
            kp = np.sort(np.concatenate([oracle.zigzag_positions(j, w.P, c) for j in range(w.P)]))
            for r in w.query_ranks:
                qp = oracle.zigzag_positions(r, w.P, c)
                pairs += int(np.searchsorted(kp, qp, side="right").sum()) if w.causal else qp.size * kp.size
        else:
            n = w.n
            for i in w.query_ranks:
                for j in range(w.P):
                    pairs += oracle.unmasked_pairs(n, n, w.causal, i * n, j * n)
        assert w.flops() == 4 * w.d * pairs * w.B * w.Hq, name


def test_aligned_score_inputs_are_sensitive():
    """The inputs of the GPU rounding-edge tests: every score of a row lies far
    above zero and the row sums of exp(score) stay well inside float range, and
    rescaling Q by log2(e) with a re-rounding to bf16 (a shortcut that skips
    the fp32 multiply of the score) moves lse past the 2e-2 bar.  So a kernel
    that took such a shortcut fails those tests; the oracle sees the inputs
    exactly as the kernel does."""
    import numpy as np
    import oracle
    from sequence_kv_chunk_amd.synth import (LOG2E_F32, aligned_score_inputs, bf16_bits_to_f32,
                                             bf16_bits_to_f64, bf16_values_rounding_down_under_log2e,
                                             f32_to_bf16_bits)
    vals, rel = bf16_values_rounding_down_under_log2e()
    x = bf16_bits_to_f64(vals)
    assert np.all((x >= 0.25) & (x < 0.5)) and np.all(rel < -2.5e-3)
    for d in (64, 128):
        q, k, v = aligned_score_inputs(1, 4, 96, 2048, d, seed=40 + d)
        qf, kf, vf = (bf16_bits_to_f64(t) for t in (q, k, v))
        _, lse = oracle.attention_fp64(qf, kf, vf)
        top = np.max(np.einsum("bhqd,bhkd->bhqk", qf, kf), axis=-1)
        assert 8.0 < top.min() and top.max() < 20.0
        log2_sum = lse / np.log(2.0)
        assert 20.0 < log2_sum.min() and log2_sum.max() < 36.0
        q_short = bf16_bits_to_f64(f32_to_bf16_bits(bf16_bits_to_f32(q) * LOG2E_F32)) / float(LOG2E_F32)
        _, lse_short = oracle.attention_fp64(q_short, kf, vf)
        assert np.max(np.abs(lse_short - lse)) > 3e-2

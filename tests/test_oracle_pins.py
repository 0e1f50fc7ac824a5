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

"""Planted mistakes in a copy of the oracle must fail at least one pin.

Each mutant copies ``oracle/`` to a temporary package, applies one textual
change of the kind a careless implementation makes (a dropped term, a wrong
sign or index, a transposed operand, an off-by-one mask), imports it, and runs
every pin.  A mutant that passes all pins would mean the pins cannot tell that
mistake from the correct oracle.
"""
import importlib
import os
import shutil
import sys

import pytest

import pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTANTS = [
    ("attention.py", "key_pos[None, :] <= qp[:, None]", "key_pos[None, :] < qp[:, None]"),
    ("attention.py", "g = h // group", "g = h % Hkv"),
    ("attention.py", "(w @ V)", "(w @ K)"),
    ("attention.py", "m + np.log(safe_l)", "m + safe_l"),
    ("attention.py", "s = scale * (q[b, h, r0:r1] @ K.T)", "s = (q[b, h, r0:r1] @ K.T)"),
    ("attention.py", "(w @ V) / safe_l[:, None]", "(w @ V)"),
    ("attention.py", "qp = q_pos0 + np.arange(r0, r1)", "qp = np.arange(r0, r1)"),
    ("attention.py", "key_pos = k_pos0 + np.arange(n_k)", "key_pos = np.arange(n_k)"),
    ("attention.py", "np.exp(s - m[:, None])", "np.exp(s)"),
    ("attention.py", "tot += max(0, min(n_k, q_pos0 + t - k_pos0 + 1))",
     "tot += max(0, min(n_k, q_pos0 + t - k_pos0))"),
    ("ring.py", "np.exp(lse_b - Ms)", "np.exp(Ms - lse_b)"),
    ("ring.py", "Ms + np.log(safe)", "Ms + safe"),
    ("ring.py", "(wb / safe)[..., None] * o_b", "(wb / safe)[..., None] * o_a"),
    ("ring.py", "(wa / safe)[..., None] * o_a", "wa[..., None] * o_a"),
    ("ring.py", "for s in range(P)]", "for s in range(max(1, P - 1))]"),
    ("ring.py", "k_pos0=j * n", "k_pos0=rank * n"),
    ("ring.py", "return [(rank - s) % P", "return [(rank + s) % P"),
    ("ulysses.py", "j = r * Hl + hl", "j = hl"),
    ("ulysses.py", "return j // (H_dst // H_src)", "return j % H_src"),
    ("ulysses.py", "dst[r, p * n:(p + 1) * n, hl, :]", "dst[p, r * n:(r + 1) * n, hl, :]"),
    ("ulysses.py", "src[r, p * n:(p + 1) * n, hl, :]", "src[p, r * n:(r + 1) * n, hl, :]"),
    ("ulysses.py", "dst[p, :, r * Hl + hl, :]", "dst[p, :, hl * P + r, :]"),
    ("closed_form.py", "L * L * elem_bytes * heads", "L * elem_bytes * heads * 1024"),
    ("attention.py", "visible = k_pos[None, :] <= q_pos[r0:r1, None]", "visible = k_pos[None, :] < q_pos[r0:r1, None]"),
    ("attention.py", "(w @ v[b, g]) / safe_l[:, None]", "(w @ v[b, h // Hkv]) / safe_l[:, None]"),
    ("zigzag.py", "late = (2 * P - 1 - rank) * c", "late = (2 * P - rank) * c"),
    ("zigzag.py", "late = (2 * P - 1 - rank) * c", "late = (P + rank) * c"),
    ("zigzag.py", "np.concatenate([early, late])", "np.concatenate([late, early])"),
    ("zigzag.py", "cls = \"full\" if kb < qa else", "cls = \"full\" if kb <= qa else"),
    ("zigzag.py", "for kb in (j, 2 * P - 1 - j):", "for kb in (j, P + j):"),
    ("zigzag.py", "zigzag_positions(rank, P, c), k_pos, scale=scale)", "zigzag_positions(rank, P, c), k_pos, scale=1.0)"),
    ("backward.py", "            dv[b, g] += p.T @ do[b, h]\n            dp = do[b, h] @ v[b, g].T\n            D = ",
     "            dv[b, g] += p @ do[b, h]\n            dp = do[b, h] @ v[b, g].T\n            D = "),
    ("backward.py", "            ds = p * (dp - D[:, None])\n            dq[b, h] = scale * (ds @ k[b, g])\n            dk[b, g] += scale * (ds.T @ q[b, h])\n    return dq, dk, dv\n\n\ndef rowsum",
     "            ds = p * dp\n            dq[b, h] = scale * (ds @ k[b, g])\n            dk[b, g] += scale * (ds.T @ q[b, h])\n    return dq, dk, dv\n\n\ndef rowsum"),
    ("backward.py", "            dq[b, h] = scale * (ds @ k[b, g])\n            dk[b, g] += scale * (ds.T @ q[b, h])\n    return dq, dk, dv\n\n\ndef rowsum",
     "            dq[b, h] = (ds @ k[b, g])\n            dk[b, g] += scale * (ds.T @ q[b, h])\n    return dq, dk, dv\n\n\ndef rowsum"),
    ("backward.py", "            dk[b, g] += scale * (ds.T @ q[b, h])\n    return dq, dk, dv\n\n\ndef rowsum",
     "            dk[b, g] = scale * (ds.T @ q[b, h])\n    return dq, dk, dv\n\n\ndef rowsum"),
    ("backward.py", "np.exp(s - np.where(fin, lse[b, h], 0.0)[:, None])", "np.exp(s - np.where(fin, lse[b, h], 0.0)[None, :])"),
    ("backward.py", "            ds = p * (dp - D[b, h][:, None])", "            ds = p * (dp - D[b, h][None, :])"),
    ("attention.py", "visible = (ids[None, :] == ids[r0:r1, None]) & (pos[None, :] <= pos[r0:r1, None])",
     "visible = (ids[None, :] <= ids[r0:r1, None]) & (pos[None, :] <= pos[r0:r1, None])"),
    ("attention.py", "        ids[s:] += 1", "        ids[s + 1:] += 1"),
    ("attention.py", "O[b, h, r0:r1] = (w @ v[b, g]) / l[:, None]", "O[b, h, r0:r1] = (w @ v[b, g])"),
    ("backward.py", "return (np.asarray(do, dtype=np.float64) * np.asarray(o, dtype=np.float64)).sum(axis=-1)",
     "return (np.asarray(do, dtype=np.float64) * np.asarray(o, dtype=np.float64)).sum(axis=-2)"),
]


def _load_copy(tmp_path, tag, fname=None, old=None, new=None):
    pkg = f"oracle_copy_{tag}"
    dst = tmp_path / pkg
    shutil.copytree(os.path.join(ROOT, "oracle"), dst)
    if fname is not None:
        p = dst / fname
        src = p.read_text()
        assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
        p.write_text(src.replace(old, new))
    sys.path.insert(0, str(tmp_path))
    try:
        importlib.invalidate_caches()
        return importlib.import_module(pkg)
    finally:
        sys.path.remove(str(tmp_path))


def _failing_pins(mod):
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(mod)
        except Exception as e:  # a pin failing in any way counts as caught
            failed.append((pin.__name__, type(e).__name__))
    return failed


def test_unmutated_copy_passes(tmp_path):
    mod = _load_copy(tmp_path, "clean")
    assert _failing_pins(mod) == []


@pytest.mark.parametrize("idx", range(len(MUTANTS)))
def test_mutant_is_caught(tmp_path, idx):
    fname, old, new = MUTANTS[idx]
    mod = _load_copy(tmp_path, f"m{idx}", fname, old, new)
    failed = _failing_pins(mod)
    assert failed, f"mutant {fname}: {old!r} -> {new!r} passed every pin"

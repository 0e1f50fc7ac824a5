"""ra_lse_merge against the oracle's log-sum-exp merge."""
import numpy as np
import pytest

import oracle

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from gpu_util import check_close, host_f64, say  # noqa: E402


@pytest.fixture(scope="module")
def api():
    from sequence_kv_chunk_amd import api
    return api


def _partials(B, H, n, d, seed):
    rng = np.random.default_rng(seed)
    oa, ob = (rng.standard_normal((B, H, n, d)).astype(np.float32) for _ in range(2))
    la, lb = (rng.standard_normal((B, H, n)).astype(np.float32) * 5 for _ in range(2))
    # empty partials: a-only, b-only and both empty rows
    la[..., 0] = -np.inf
    oa[..., 0, :] = 0
    lb[..., 1] = -np.inf
    ob[..., 1, :] = 0
    la[..., 2] = lb[..., 2] = -np.inf
    oa[..., 2, :] = ob[..., 2, :] = 0
    lb[..., 3] = la[..., 3] + 40.0   # one side dominates completely
    return oa, la, ob, lb


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dts", [("f32", "f32", "f32"), ("f32", "f32", "bf16"), ("bf16", "f32", "f32"),
                                 ("bf16", "bf16", "bf16")])
def test_merge_matches_oracle(api, d, dts):
    B, H, n = 2, 3, 77
    say(f"merge d={d} {dts}")
    oa, la, ob, lb = _partials(B, H, n, d, seed=d)
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16}
    ta = torch.from_numpy(oa).cuda().to(tdt[dts[0]])
    tb = torch.from_numpy(ob).cuda().to(tdt[dts[1]])
    oa_x, ob_x = host_f64(ta), host_f64(tb)     # what the kernel actually receives
    ref_o, ref_l = oracle.lse_merge_fp64(oa_x, la, ob_x, lb)
    to = torch.full((B, H, n, d), float("nan"), device="cuda").to(tdt[dts[2]])
    tl = torch.full((B * H * n,), float("nan"), device="cuda")
    api.ra_lse_merge(ta, torch.from_numpy(la).cuda().reshape(-1), tb, torch.from_numpy(lb).cuda().reshape(-1),
                     to, tl)
    torch.cuda.synchronize()
    tol = "bf16" if "bf16" in dts else "f32"
    check_close(host_f64(to), ref_o, tol, "O")
    check_close(host_f64(tl).reshape(B, H, n), ref_l, tol, "lse")


@pytest.mark.parametrize("into", ["a", "b"])
def test_merge_in_place(api, into):
    B, H, n, d = 1, 4, 130, 128
    oa, la, ob, lb = _partials(B, H, n, d, seed=3)
    ref_o, ref_l = oracle.lse_merge_fp64(oa, la, ob, lb)
    ta, tb = torch.from_numpy(oa).cuda(), torch.from_numpy(ob).cuda()
    tla, tlb = torch.from_numpy(la).cuda().reshape(-1), torch.from_numpy(lb).cuda().reshape(-1)
    to, tl = (ta, tla) if into == "a" else (tb, tlb)
    api.ra_lse_merge(ta, tla, tb, tlb, to, tl)
    torch.cuda.synchronize()
    check_close(host_f64(to), ref_o, "f32", "O")
    check_close(host_f64(tl).reshape(B, H, n), ref_l, "f32", "lse")


def test_merge_strided_views(api):
    # [S, H, d] layouts (a Ulysses share) merge through strided views
    S, H, d = 100, 4, 64
    rng = np.random.default_rng(4)
    oa, ob = (rng.standard_normal((S, H, d)).astype(np.float32) for _ in range(2))
    la, lb = (rng.standard_normal((H, S)).astype(np.float32) for _ in range(2))
    ref_o, ref_l = oracle.lse_merge_fp64(oa.transpose(1, 0, 2), la, ob.transpose(1, 0, 2), lb)
    ta, tb = torch.from_numpy(oa).cuda(), torch.from_numpy(ob).cuda()
    to = torch.empty_like(ta)
    tl = torch.empty(H * S, device="cuda")
    api.ra_lse_merge(ta, torch.from_numpy(la).cuda().reshape(-1), tb, torch.from_numpy(lb).cuda().reshape(-1),
                     to, tl)
    torch.cuda.synchronize()
    check_close(host_f64(to).transpose(1, 0, 2), ref_o, "f32", "O")
    check_close(host_f64(tl).reshape(H, S), ref_l, "f32", "lse")

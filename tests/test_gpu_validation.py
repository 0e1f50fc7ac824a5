"""The host-side argument checks of the C ABI, on a machine with a GPU: the
cases of test_abi_cpu.py with every address inside one real 10 GiB device
allocation (the cases use offsets below 9.1 GiB).  Every case is invalid, so
each call must return its error status before any HIP call; and should a check
ever let one through, its kernel would still only touch that allocation."""
import pytest

import test_abi_cpu as cases

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from gpu_util import say  # noqa: E402


@pytest.fixture(scope="module")
def lib():
    import ctypes
    return ctypes.CDLL(cases.LIB)


@pytest.fixture(scope="module")
def real_base():
    buf = torch.empty(10 << 30, dtype=torch.uint8, device="cuda")
    old = cases.BASE
    cases.BASE = buf.data_ptr()
    say(f"validation cases on a real allocation at {cases.BASE:#x}")
    yield buf
    cases.BASE = old
    torch.cuda.synchronize()
    del buf
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name,kw,want", cases.ATTN_BAD, ids=[c[0] for c in cases.ATTN_BAD])
def test_chunk_attention_rejects(real_base, lib, name, kw, want):
    cases.check_attn_case(lib, name, kw, want)


@pytest.mark.parametrize("check", ["ring", "zigzag", "usp", "merge", "ulysses", "bwd", "bwd_preprocess", "ring_bwd", "empty"])
def test_entry_points_reject(real_base, lib, check):
    getattr(cases, f"check_{check}")(lib)
    torch.cuda.synchronize()

"""reduce_axis0_split_noalloc: the split column sum with its float64 partials
in the library's static device array instead of a caller workspace.

Checked through the C ABI against reduce_axis0_split with a workspace (the
same kernels and chunking, so the same bits), on consecutive calls whose
second input is smaller than the first -- the static array keeps the previous
call's partials, and every partial the second call reads must be its own --
and exactly against integer column sums.  Neither the binding nor the library
allocates: torch's allocator counters do not move across the calls.
"""
import numpy as np
import pytest

from parity_util import host, say
from cfc_recurrent_cell_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests selected but torch sees no GPU")
    import cfc_recurrent_cell_amd as C
    C.load_library()
    return torch.device("cuda:0")


def _with_workspace(t):
    import torch
    import cfc_recurrent_cell_amd as C
    B, N = t.shape
    ws = torch.empty((max(1, C.reduce_axis0_split_workspace(B, N)),), dtype=torch.uint8, device="cuda")
    return C.reduce_axis0(t, split=True, workspace=ws)


@pytest.mark.parametrize("shapes", [((524288, 3), (20000, 3)), ((65536, 200), (9000, 37)),
                                    ((262144, 64), (131072, 64))],
                         ids=["N3", "N200_then_N37", "N64"])
def test_noalloc_matches_workspace_entry_on_consecutive_calls(shapes):
    import torch
    import cfc_recurrent_cell_amd as C
    inputs = []
    for i, (B, N) in enumerate(shapes):
        a = W.make_random_matrix(B, N, seed=4000 + i)
        inputs.append(torch.from_numpy(a).cuda())
    outs = [torch.full((t.shape[1],), float("nan"), device="cuda") for t in inputs]
    torch.cuda.synchronize()
    before = (torch.cuda.memory_allocated(), torch.cuda.memory_stats().get("allocation.all.allocated", 0))
    for t, o in zip(inputs, outs):          # two calls in a row, the second smaller
        say(f"[no-alloc] B={t.shape[0]} N={t.shape[1]}")
        C.reduce_axis0_noalloc(t, o)
    torch.cuda.synchronize()
    after = (torch.cuda.memory_allocated(), torch.cuda.memory_stats().get("allocation.all.allocated", 0))
    assert before == after, "the allocation-free call allocated device memory through torch"
    for t, o in zip(inputs, outs):
        ref = _with_workspace(t)
        assert np.array_equal(host(o).view(np.uint32), host(ref).view(np.uint32)), \
            f"B={t.shape[0]} N={t.shape[1]}: differs from reduce_axis0_split with a workspace"


def test_noalloc_integer_sums_are_exact():
    import torch
    import cfc_recurrent_cell_amd as C
    for B, N, seed in ((300000, 5, 4101), (70000, 256, 4102)):
        a = W.make_random_matrix(B, N, seed=seed, integer=True)
        say(f"[no-alloc] integers B={B} N={N}")
        out = torch.full((N,), float("nan"), device="cuda")
        C.reduce_axis0_noalloc(torch.from_numpy(a).cuda(), out)
        assert np.array_equal(host(out).astype(np.int64), a.astype(np.int64).sum(0))


def test_noalloc_without_a_split_is_the_one_pass_reduce():
    """Shapes the split plan does not split (N > 256, or few rows) take the
    one-pass reduce_axis0, as reduce_axis0_split does."""
    import torch
    import cfc_recurrent_cell_amd as C
    for B, N in ((40, 1000), (10, 3), (0, 7)):
        a = W.make_random_matrix(B, N, seed=4200 + N)
        t = torch.from_numpy(a).cuda()
        out = torch.full((N,), float("nan"), device="cuda")
        C.reduce_axis0_noalloc(t, out)
        ref = C.reduce_axis0(t)
        assert np.array_equal(host(out).view(np.uint32), host(ref).view(np.uint32))

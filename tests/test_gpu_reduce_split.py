"""GPU checks of reduce_axis0_split (narrow rows over a long leading axis,
two phases through a caller workspace) and of merged leading axes, through the
C ABI.  Integer-valued inputs make every partial sum exact in float32 and
float64, so the result must equal the exact integer column sum bitwise;
real-valued inputs must be within one float32 ulp of the float64 sum of the
same float32 rows (the oracle's column sum).
"""
import numpy as np
import pytest

from parity_util import host, say
from oracle import oracle as O
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


def _within_one_ulp(got, a_f32, what):
    own = O.reduce_axis0_f32(a_f32)
    diff = np.abs(got.astype(np.float64) - own)
    ulp = np.spacing(np.abs(own.astype(np.float32))).astype(np.float64)
    bad = np.flatnonzero(diff > ulp)
    assert bad.size == 0, f"{what}: {bad.size} columns more than 1 ulp from the float64 sum, first {bad[:5]}"


# the pages' case (3 outputs over B*Q = 524288 rows) and other narrow widths
SHAPES = [(524288, 3), (100000, 1), (300001, 7), (65536, 64), (20000, 200), (20000, 256), (5003, 33),
          (1100, 2)]


@pytest.mark.parametrize("B,N", SHAPES)
def test_split_reduce_integer_exact(B, N):
    import torch
    import cfc_recurrent_cell_amd as C
    say(f"[split reduce] integer B={B} N={N} workspace={C.reduce_axis0_split_workspace(B, N)} bytes")
    assert C.reduce_axis0_split_workspace(B, N) > 0
    a = W.make_random_matrix(B, N, seed=B + 7 * N, integer=True)
    t = torch.from_numpy(a).cuda()
    out = torch.full((N,), float("nan"), device="cuda")
    C.reduce_axis0(t, out=out, split=True)
    g = host(out)
    assert np.array_equal(g.astype(np.int64), a.astype(np.int64).sum(axis=0))


@pytest.mark.parametrize("B,N", [(524288, 3), (65536, 64), (20000, 256)])
def test_split_reduce_real_valued_and_deterministic(B, N):
    import torch
    import cfc_recurrent_cell_amd as C
    say(f"[split reduce] real B={B} N={N}")
    a = W.make_random_matrix(B, N, seed=3 * B + N)
    t = torch.from_numpy(a).cuda()
    ws = torch.empty((C.reduce_axis0_split_workspace(B, N),), dtype=torch.uint8, device="cuda")
    first = host(C.reduce_axis0(t, split=True, workspace=ws)).copy()
    _within_one_ulp(first, a, f"split B={B} N={N}")
    ws.fill_(0xFF)   # NaN bytes: the workspace's contents on entry do not matter
    again = host(C.reduce_axis0(t, split=True, workspace=ws))
    assert np.array_equal(first.view(np.uint32), again.view(np.uint32))


@pytest.mark.parametrize("B,N", [(10, 3), (7, 200), (1000, 300), (0, 5)])
def test_split_reduce_falls_back_to_one_pass(B, N):
    """Too few rows to split, or wider than 256: no workspace, same bits as
    reduce_axis0."""
    import torch
    import cfc_recurrent_cell_amd as C
    assert C.reduce_axis0_split_workspace(B, N) == 0
    a = W.make_random_matrix(B, N, seed=11 + B + N)
    t = torch.from_numpy(a).cuda()
    g = host(C.reduce_axis0(t, split=True))
    r = host(C.reduce_axis0(t))
    assert np.array_equal(g.view(np.uint32), r.view(np.uint32))
    if B == 0:
        assert np.array_equal(g, np.zeros(N, np.float32))


@pytest.mark.parametrize("split", [False, True])
def test_merged_leading_axes(split):
    """A [B, heads, E, H] scratch reduced over batch and heads: the two leading
    axes merge into the reduced axis, the rest into the columns, and the
    result has the trailing shape."""
    import torch
    import cfc_recurrent_cell_amd as C
    a = W.make_random_matrix(4096 * 4, 2 * 3 * 5, seed=99, integer=True).reshape(4096, 4, 2, 15)
    say(f"[merged axes] split={split}")
    t = torch.from_numpy(np.ascontiguousarray(a)).cuda()
    out = C.reduce_axis0(t, leading_axes=2, split=split)
    assert tuple(out.shape) == (2, 15)
    assert np.array_equal(host(out).astype(np.int64), a.astype(np.int64).sum(axis=(0, 1)))
    out3 = C.reduce_axis0(t, leading_axes=3, split=split)
    assert tuple(out3.shape) == (15,)
    assert np.array_equal(host(out3).astype(np.int64), a.astype(np.int64).sum(axis=(0, 1, 2)))

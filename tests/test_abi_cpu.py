"""C-ABI checks that need no GPU: the library loads, exports every declared
symbol, and rejects bad arguments with the documented codes before it
touches the HIP runtime (so none of these calls enqueues anything)."""
import ctypes
import os

import pytest

import cfc_recurrent_cell_amd as C
from cfc_recurrent_cell_amd import _lib

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH),
                                reason="libcfc_amd.so not built (run __graft_entry__.build())")

FAKE = 0x10000          # never dereferenced: every call below fails validation first


def _params(n_in=8, n_hid=16, base=FAKE, cell=0):
    return C.CfcParams(base, base + 0x100000, base + 0x200000, base + 0x300000, n_in, n_hid, cell)


@pytest.fixture(scope="module")
def lib():
    return C.load_library()


def test_exports_every_declared_symbol(lib):
    names = _lib.declared_symbols()
    assert set(names) == {"cfc_scratch_row_len", "cfc_forward", "cfc_backward", "cfc_backward_window",
                          "cfc_forward_backward", "reduce_axis0", "reduce_axis0_split",
                          "reduce_axis0_split_workspace", "cfc_status_string", "cfc_backward_workspace",
                          "cfc_backward_window_ws", "cfc_forward_backward_ws", "reduce_axis0_split_noalloc",
                          "cfc_forward_backward_workspace"}
    for n in names:
        assert hasattr(lib, n), n


def test_scratch_row_len(lib):
    assert lib.cfc_scratch_row_len(16, 32) == 32 * (16 + 32 + 2) == 1600
    assert lib.cfc_scratch_row_len(128, 128) == 33024
    assert lib.cfc_scratch_row_len(256, 256) == 131584
    assert lib.cfc_scratch_row_len(0, 4) == -1
    assert lib.cfc_scratch_row_len(4, -1) == -1
    assert lib.cfc_scratch_row_len(2**31 - 1, 2**31 - 1) == -1     # overflow


def test_status_strings(lib):
    for code in range(7):
        assert lib.cfc_status_string(code)
    assert lib.cfc_status_string(99) == b"unknown status code"


def _fwd(lib, p, x=FAKE + 0x400000, h0=FAKE + 0x500000, dt=1.0, B=2, K=3, h_seq=FAKE + 0x600000):
    return lib.cfc_forward(ctypes.byref(p) if p is not None else None, x, h0, dt, B, K, h_seq, None)


def _bwd(lib, p, dt=1.0, B=2, K=3, flags=0, scratch=FAKE + 0x900000, loss=None, h_seq=FAKE + 0x600000,
         grad_x=None, grad_h0=None):
    return lib.cfc_backward(ctypes.byref(p) if p is not None else None, FAKE + 0x400000,
                            FAKE + 0x500000, h_seq, FAKE + 0x700000, dt, B, K, scratch, loss,
                            grad_x, grad_h0, flags, None)


def test_forward_validation(lib):
    assert _fwd(lib, None) == C.CFC_ERR_NULL
    p = _params()
    p.w_rec = None
    assert _fwd(lib, p) == C.CFC_ERR_NULL
    assert _fwd(lib, _params(), x=None) == C.CFC_ERR_NULL
    assert _fwd(lib, _params(), h_seq=None) == C.CFC_ERR_NULL
    assert _fwd(lib, _params(n_in=0)) == C.CFC_ERR_DIM
    assert _fwd(lib, _params(n_hid=-3)) == C.CFC_ERR_DIM
    assert _fwd(lib, _params(), B=0) == C.CFC_ERR_DIM
    assert _fwd(lib, _params(), K=0) == C.CFC_ERR_DIM
    assert _fwd(lib, _params(), dt=float("nan")) == C.CFC_ERR_DT
    assert _fwd(lib, _params(), dt=float("inf")) == C.CFC_ERR_DT
    assert _fwd(lib, _params(n_in=257)) == C.CFC_ERR_UNSUPPORTED
    assert _fwd(lib, _params(n_hid=300)) == C.CFC_ERR_UNSUPPORTED
    # unknown cell type
    assert _fwd(lib, _params(cell=2)) == C.CFC_ERR_UNSUPPORTED
    assert _fwd(lib, _params(cell=-1)) == C.CFC_ERR_UNSUPPORTED
    # output overlapping an input: h_seq [2,3,16] starting inside x
    assert _fwd(lib, _params(), h_seq=FAKE + 0x400000 + 8) == C.CFC_ERR_OVERLAP
    # h_seq overlapping the weights
    assert _fwd(lib, _params(), h_seq=FAKE + 0x100000 - 4) == C.CFC_ERR_OVERLAP


def test_backward_validation(lib):
    assert _bwd(lib, None) == C.CFC_ERR_NULL
    assert _bwd(lib, _params(), scratch=None) == C.CFC_ERR_NULL
    assert _bwd(lib, _params(), B=0) == C.CFC_ERR_DIM
    assert _bwd(lib, _params(), flags=7) == C.CFC_ERR_DIM
    assert _bwd(lib, _params(), dt=float("-inf")) == C.CFC_ERR_DT
    assert _bwd(lib, _params(n_in=512)) == C.CFC_ERR_UNSUPPORTED
    assert _bwd(lib, _params(cell=7)) == C.CFC_ERR_UNSUPPORTED
    # LDS bound: K * (12 H + 4 n_in) + 40 H + 2048 <= 160 KiB
    assert _bwd(lib, _params(n_in=128, n_hid=128), K=77) == C.CFC_ERR_UNSUPPORTED
    assert _bwd(lib, _params(n_in=256, n_hid=256), K=38) == C.CFC_ERR_UNSUPPORTED
    # scratch overlapping h_seq
    assert _bwd(lib, _params(), scratch=FAKE + 0x600000 + 64) == C.CFC_ERR_OVERLAP
    # loss overlapping scratch
    assert _bwd(lib, _params(), loss=FAKE + 0x900000 + 4) == C.CFC_ERR_OVERLAP
    # input gradients: grad_x [2,3,8] over x, over scratch; grad_h0 [2,16] over y, over grad_x
    assert _bwd(lib, _params(), grad_x=FAKE + 0x400000) == C.CFC_ERR_OVERLAP
    assert _bwd(lib, _params(), grad_x=FAKE + 0x900000 + 8) == C.CFC_ERR_OVERLAP
    assert _bwd(lib, _params(), grad_h0=FAKE + 0x700000 + 4) == C.CFC_ERR_OVERLAP
    assert _bwd(lib, _params(), grad_x=FAKE + 0xA00000, grad_h0=FAKE + 0xA00000 + 16) == C.CFC_ERR_OVERLAP


def _fb(lib, p, dt=1.0, B=2, K=3, flags=0, h_seq=FAKE + 0x600000, scratch=FAKE + 0x900000, loss=None,
        y=FAKE + 0x700000, grad_x=None, grad_h0=None):
    return lib.cfc_forward_backward(ctypes.byref(p) if p is not None else None, FAKE + 0x400000,
                                    FAKE + 0x500000, y, dt, B, K, h_seq, scratch, loss, grad_x, grad_h0,
                                    flags, None)


def test_forward_backward_validation(lib):
    """The one-call path applies the rules of both directions before it
    enqueues anything, including the backward's LDS limit on the shapes that
    fall back to two launches."""
    assert _fb(lib, None) == C.CFC_ERR_NULL
    assert _fb(lib, _params(), y=None) == C.CFC_ERR_NULL
    assert _fb(lib, _params(), h_seq=None) == C.CFC_ERR_NULL
    assert _fb(lib, _params(), scratch=None) == C.CFC_ERR_NULL
    assert _fb(lib, _params(), B=0) == C.CFC_ERR_DIM
    assert _fb(lib, _params(), K=0) == C.CFC_ERR_DIM
    assert _fb(lib, _params(), flags=2) == C.CFC_ERR_DIM
    assert _fb(lib, _params(), dt=float("nan")) == C.CFC_ERR_DT
    assert _fb(lib, _params(n_hid=257)) == C.CFC_ERR_UNSUPPORTED
    assert _fb(lib, _params(cell=3)) == C.CFC_ERR_UNSUPPORTED
    assert _fb(lib, _params(n_in=128, n_hid=128), K=77) == C.CFC_ERR_UNSUPPORTED
    assert _fb(lib, _params(n_in=256, n_hid=256), K=38) == C.CFC_ERR_UNSUPPORTED
    # outputs against inputs, and against each other
    assert _fb(lib, _params(), h_seq=FAKE + 0x400000 + 8) == C.CFC_ERR_OVERLAP
    assert _fb(lib, _params(), scratch=FAKE + 0x700000) == C.CFC_ERR_OVERLAP
    assert _fb(lib, _params(), scratch=FAKE + 0x600000 + 64) == C.CFC_ERR_OVERLAP
    assert _fb(lib, _params(), loss=FAKE + 0x600000 + 4) == C.CFC_ERR_OVERLAP
    assert _fb(lib, _params(), loss=FAKE + 0x900000 + 4) == C.CFC_ERR_OVERLAP
    assert _fb(lib, _params(), grad_x=FAKE + 0x600000 + 4) == C.CFC_ERR_OVERLAP
    assert _fb(lib, _params(), grad_h0=FAKE + 0x500000) == C.CFC_ERR_OVERLAP


def _win(lib, p, k_begin, k_end, K=6, y=FAKE + 0x700000, delta_in=None, delta_out=None, loss=None, flags=0,
         scratch=FAKE + 0x900000):
    return lib.cfc_backward_window(ctypes.byref(p), FAKE + 0x400000, FAKE + 0x500000, FAKE + 0x600000, y,
                                   delta_in, 1.0, 2, K, k_begin, k_end, scratch, loss, None, delta_out, flags,
                                   None)


def test_backward_window_validation(lib):
    p = _params()
    D1, D2 = FAKE + 0xB00000, FAKE + 0xC00000
    assert _win(lib, p, 2, 2) == C.CFC_ERR_DIM            # empty window
    assert _win(lib, p, 3, 2) == C.CFC_ERR_DIM
    assert _win(lib, p, -1, 6) == C.CFC_ERR_DIM
    assert _win(lib, p, 0, 7) == C.CFC_ERR_DIM            # past K
    assert _win(lib, p, 0, 4) == C.CFC_ERR_DIM            # seeded from y but not ending at K
    assert _win(lib, p, 0, 6, y=None) == C.CFC_ERR_NULL   # no seed at all
    assert _win(lib, p, 0, 4, y=None, delta_in=D1, loss=FAKE + 0xD00000) == C.CFC_ERR_DIM  # loss without seed
    assert _win(lib, p, 0, 4, y=None, delta_in=D1, flags=5) == C.CFC_ERR_DIM
    # delta_out partly over delta_in ([2,16] floats), or over the scratch
    assert _win(lib, p, 0, 4, y=None, delta_in=D1, delta_out=D1 + 8) == C.CFC_ERR_OVERLAP
    assert _win(lib, p, 0, 4, y=None, delta_in=D1, delta_out=FAKE + 0x900000 + 4) == C.CFC_ERR_OVERLAP
    # delta_in over an output
    assert _win(lib, p, 0, 4, y=None, delta_in=FAKE + 0x900000, delta_out=D2) == C.CFC_ERR_OVERLAP
    # the window's own LDS bound: 64 steps of 128/128 fit, 77 do not
    big = _params(n_in=128, n_hid=128)
    assert _win(lib, big, 0, 77, K=200, y=None, delta_in=D1) == C.CFC_ERR_UNSUPPORTED


def test_backward_workspace_sizes(lib):
    """8 B Kw n_hid bytes (dL/da of every row-step in float64) where the
    16-row backward runs in accumulate mode, 0 elsewhere."""
    ws = lib.cfc_backward_workspace
    assert ws(8192, 8, 256, 256, C.CFC_ACCUMULATE) == 8 * 8192 * 8 * 256
    assert ws(3, 20, 129, 7, C.CFC_ACCUMULATE) == 8 * 3 * 20 * 7       # n_in alone above 128
    assert ws(3, 20, 7, 129, C.CFC_ACCUMULATE) == 8 * 3 * 20 * 129
    assert ws(3, 21, 256, 256, C.CFC_ACCUMULATE) == 0                  # beyond 20 steps: general kernel
    assert ws(3, 8, 256, 256, C.CFC_OVERWRITE) == 0                    # overwrite parks in the scratch
    assert ws(3, 64, 128, 128, C.CFC_ACCUMULATE) == 0                  # one-row kernels keep dL/da on chip
    assert ws(0, 8, 256, 256, C.CFC_ACCUMULATE) == -1
    assert ws(3, 0, 256, 256, C.CFC_ACCUMULATE) == -1
    assert ws(3, 8, 0, 256, C.CFC_ACCUMULATE) == -1
    assert ws(3, 8, 256, 256, 7) == -1
    assert ws(2**31 - 1, 20, 256, 2**31 - 1, C.CFC_ACCUMULATE) == -1   # overflow


def test_forward_backward_workspace_sizes(lib):
    """The one-call entry's size: the backward's, plus the 1 MiB float64 weight
    copy (2 x 256 x 256 doubles) at exactly 256 x 256 with K <= 8 in
    accumulate mode."""
    fb, bw = lib.cfc_forward_backward_workspace, lib.cfc_backward_workspace
    A = C.CFC_ACCUMULATE
    assert fb(8192, 8, 256, 256, A) == 8 * 8192 * 8 * 256 + 2 * 256 * 256 * 8
    assert fb(3, 1, 256, 256, A) == bw(3, 1, 256, 256, A) + (1 << 20)
    for args in ((3, 9, 256, 256, A), (3, 8, 200, 256, A), (3, 8, 256, 200, A), (3, 8, 256, 256, C.CFC_OVERWRITE),
                 (3, 64, 128, 128, A), (3, 21, 256, 256, A), (0, 8, 256, 256, A), (3, 8, 256, 256, 7)):
        assert fb(*args) == bw(*args), args


def _win_ws(lib, p, ws, ws_bytes, k_begin=0, k_end=6, K=6, flags=C.CFC_ACCUMULATE, scratch=FAKE + 0x900000):
    return lib.cfc_backward_window_ws(ctypes.byref(p), FAKE + 0x400000, FAKE + 0x500000, FAKE + 0x600000,
                                      FAKE + 0x700000, None, 1.0, 2, K, k_begin, k_end, scratch, None, None, None,
                                      flags, ws, ws_bytes, None)


def test_backward_window_ws_validation(lib):
    """The workspace is checked where the window would use it: size, 8-byte
    alignment, overlap with every other argument.  Every call here fails
    validation, so none launches anything."""
    p = _params(n_in=256, n_hid=256)                     # scratch [2, 131584] at FAKE + 0x900000 (1 MB)
    need = 8 * 2 * 6 * 256
    WS = FAKE + 0x1000000
    assert _win_ws(lib, p, WS, need - 1) == C.CFC_ERR_DIM            # too small
    assert _win_ws(lib, p, WS + 4, need) == C.CFC_ERR_DIM            # misaligned
    assert _win_ws(lib, p, FAKE + 0x900000 + 64, need) == C.CFC_ERR_OVERLAP   # over the scratch
    assert _win_ws(lib, p, FAKE + 0x400000, need) == C.CFC_ERR_OVERLAP        # over x
    assert _win_ws(lib, p, FAKE + 0x100000, need) == C.CFC_ERR_OVERLAP        # over W_in
    # the cfc_backward_window checks still come first
    assert _win_ws(lib, p, WS, need, k_begin=0, k_end=4) == C.CFC_ERR_DIM      # seeded, not ending at K
    assert _win_ws(lib, p, WS, need, flags=9) == C.CFC_ERR_DIM
    # a window of 7 steps needs more than a 6-step workspace
    assert _win_ws(lib, p, WS, need, K=7, k_end=7) == C.CFC_ERR_DIM


def test_forward_backward_ws_validation(lib):
    """The one-call entry checks the workspace before it enqueues the
    forward: size, alignment, overlap (with h_seq too)."""
    p = _params(n_in=256, n_hid=256)
    need = 8 * 2 * 6 * 256
    WS = FAKE + 0x1000000

    def fbw(ws, nbytes, flags=C.CFC_ACCUMULATE):
        return lib.cfc_forward_backward_ws(ctypes.byref(p), FAKE + 0x400000, FAKE + 0x500000, FAKE + 0x700000,
                                           1.0, 2, 6, FAKE + 0x600000, FAKE + 0x900000, None, None, None, flags,
                                           ws, nbytes, None)
    assert fbw(WS, need - 1) == C.CFC_ERR_DIM
    assert fbw(WS + 4, need) == C.CFC_ERR_DIM
    # with room for the float64 weight copy the whole size is checked for
    # overlap: this workspace ends 32 KB before the scratch, its copy would not
    full = lib.cfc_forward_backward_workspace(2, 6, 256, 256, C.CFC_ACCUMULATE)
    assert full == need + (1 << 20)
    near = FAKE + 0x900000 - 0x8000
    assert fbw(near, full) == C.CFC_ERR_OVERLAP
    assert fbw(FAKE + 0x600000, need) == C.CFC_ERR_OVERLAP     # over h_seq
    assert fbw(FAKE + 0x900000, need) == C.CFC_ERR_OVERLAP     # over the scratch
    assert fbw(FAKE + 0x200000, need) == C.CFC_ERR_OVERLAP     # over b
    assert fbw(WS, need, flags=3) == C.CFC_ERR_DIM


def test_backward_lds_limit_matches_header(lib):
    """The documented K limits are exactly where the library starts refusing."""
    def lds(K, n_in, H):
        return K * (12 * H + 4 * n_in) + 40 * H + 2048
    for n_in, H, kmax in ((128, 128, 76), (256, 256, 37)):
        assert lds(kmax, n_in, H) <= 160 * 1024 < lds(kmax + 1, n_in, H)


def test_reduce_validation(lib):
    assert lib.reduce_axis0(FAKE, -1, 4, FAKE + 0x100000, None) == C.CFC_ERR_DIM
    assert lib.reduce_axis0(FAKE, 4, -1, FAKE + 0x100000, None) == C.CFC_ERR_DIM
    assert lib.reduce_axis0(FAKE, 2**40, 2**40, FAKE + 0x100000, None) == C.CFC_ERR_DIM
    assert lib.reduce_axis0(FAKE, 4, 0, None, None) == C.CFC_OK          # N = 0: nothing to do
    assert lib.reduce_axis0(None, 4, 8, FAKE, None) == C.CFC_ERR_NULL
    assert lib.reduce_axis0(FAKE, 4, 8, None, None) == C.CFC_ERR_NULL
    assert lib.reduce_axis0(FAKE, 4, 8, FAKE + 16, None) == C.CFC_ERR_OVERLAP


def test_split_reduce_workspace_sizes(lib):
    """Chunking depends only on (B, N): 256 // N rows per pass, at least 8
    passes per chunk, at most 1024 chunks and 256 K partials."""
    ws = lib.reduce_axis0_split_workspace
    # N = 3: 85 rows per pass, chunks of max(ceil(524288/1024), 680) = 680 rows -> 772 chunks
    assert ws(524288, 3) == 772 * 3 * 8
    assert ws(10, 3) == 0                    # one chunk: the one-pass reduce runs
    assert ws(100000, 300) == 0              # wider than 256: one pass
    assert ws(100000, 0) == 0
    assert ws(-1, 3) == -1 and ws(3, -1) == -1
    assert ws(2**40, 2**40) == -1            # B*N*4 overflows
    # N = 256: one row per pass, at least 8-row chunks, 1024 chunks at most
    # (256 K partials): 20000 rows -> chunks of ceil(20000/1024) = 20 rows -> 1000 chunks
    assert ws(20000, 256) == 1000 * 256 * 8
    # N = 200: one row per pass, 1024 chunks at most (1310 by the partials cap):
    # 300000 rows -> chunks of ceil(300000/1024) = 293 rows -> 1024 chunks
    assert ws(300000, 200) == 1024 * 200 * 8
    assert ws(2048, 256) == 256 * 256 * 8
    assert ws(16, 256) == 2 * 256 * 8


def test_split_reduce_validation(lib):
    big = FAKE + 0x10000000
    f = lib.reduce_axis0_split
    assert f(FAKE, 524288, 3, big, None, 0, None) == C.CFC_ERR_NULL          # workspace needed
    assert f(None, 524288, 3, big, big + 0x100000, 18528, None) == C.CFC_ERR_NULL
    assert f(FAKE, 524288, 3, big, big + 0x100000, 18527, None) == C.CFC_ERR_DIM   # too small
    assert f(FAKE, 524288, 3, big, big + 0x100004, 18528, None) == C.CFC_ERR_DIM   # misaligned
    assert f(FAKE, 524288, 3, big, FAKE + 64, 18528, None) == C.CFC_ERR_OVERLAP    # over the input
    assert f(FAKE, 524288, 3, big, big + 8, 18528, None) == C.CFC_ERR_OVERLAP      # over out
    assert f(FAKE, -5, 3, big, None, 0, None) == C.CFC_ERR_DIM


def test_split_reduce_noalloc_validation(lib):
    """Argument errors of the allocation-free split reduce are reported before
    the static array's address is resolved (no HIP call)."""
    big = FAKE + 0x10000000
    f = lib.reduce_axis0_split_noalloc
    assert f(FAKE, 524288, 3, None, None) == C.CFC_ERR_NULL
    assert f(None, 524288, 3, big, None) == C.CFC_ERR_NULL
    assert f(FAKE, 524288, 3, FAKE + 64, None) == C.CFC_ERR_OVERLAP     # out over the input
    assert f(FAKE, -5, 3, big, None) == C.CFC_ERR_DIM
    assert f(FAKE, 2**40, 2**40, big, None) == C.CFC_ERR_DIM            # B*N*4 overflows
    # the largest split plan fits the static array
    worst = max(lib.reduce_axis0_split_workspace(B, N) for N in range(1, 257)
                for B in (2**20, 2**26, 3 * 2**30 // N))
    assert 0 < worst <= 2 * 1024 * 1024


def test_reduce_binding_checks_leading_axes():
    import torch
    t = torch.zeros(2, 3, 4)
    with pytest.raises(ValueError, match="leading_axes"):
        C.reduce_axis0(t, leading_axes=0)
    with pytest.raises(ValueError, match="leading_axes"):
        C.reduce_axis0(t, leading_axes=4)


def test_python_binding_rejects_unknown_cell():
    import torch
    t = torch.zeros(4)
    with pytest.raises(ValueError, match="cell must be one of"):
        C.cfc_forward(t.view(2, 2), t.view(2, 2), t[:2], t[:2], t.view(1, 1, 4), t.view(2, 2)[:1], 1.0,
                      cell="leaky")


def test_product_path_never_imports_the_oracle():
    import sys
    import subprocess
    code = ("import sys, cfc_recurrent_cell_amd as C; C.load_library(); "
            "assert not any(m == 'oracle' or m.startswith('oracle.') for m in sys.modules)")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    subprocess.run([sys.executable, "-c", code], check=True, cwd=root)

"""ctypes wrapper around ``cfc_oracle.c`` (TEST INFRASTRUCTURE ONLY).

The C file is the oracle; this module only builds it with gcc, widens float32
inputs to float64 and marshals numpy arrays.  Row ranges can be evaluated in
parallel threads (ctypes releases the GIL), which is how the large workload's
oracle finishes in tolerable time: rows are independent, so the result does
not depend on how rows are split.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "cfc_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
CELLS = {"gated": 0, "tau_decay": 1}   # the oracle's cell codes
_fp = ctypes.POINTER(ctypes.c_float)


def build_oracle(src: str = _SRC, out: str = _LIB) -> str:
    """Compile the oracle with plain gcc: -O2, no fast-math, no FMA contraction."""
    cmd = ["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
           "-shared", "-o", out, src, "-lm"]
    subprocess.run(cmd, check=True)
    return out


def _bind(lib):
    lib.oracle_scratch_row_len.restype = ctypes.c_longlong
    lib.oracle_scratch_row_len.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.oracle_cfc_forward.restype = ctypes.c_int
    lib.oracle_cfc_forward.argtypes = [ctypes.c_int] * 4 + [ctypes.c_double] + [_dp] * 7 + [ctypes.c_int]
    lib.oracle_cfc_backward_inputs.restype = ctypes.c_int
    lib.oracle_cfc_backward_inputs.argtypes = [ctypes.c_int] * 4 + [ctypes.c_double] + [_dp] * 12 + [ctypes.c_int]
    lib.oracle_reduce_axis0.restype = ctypes.c_int
    lib.oracle_reduce_axis0.argtypes = [ctypes.c_longlong, ctypes.c_longlong, _dp, _dp]
    lib.oracle_reduce_axis0_f32.restype = ctypes.c_int
    lib.oracle_reduce_axis0_f32.argtypes = [ctypes.c_longlong, ctypes.c_longlong, _fp, _dp]
    return lib


def load_oracle(path: Optional[str] = None):
    """Load (building first if absent) the oracle library."""
    global _lib
    with _lock:
        if path is not None:
            return _bind(ctypes.CDLL(path))
        if _lib is None:
            if (not os.path.exists(_LIB)) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build_oracle()
            _lib = _bind(ctypes.CDLL(_LIB))
        return _lib


def _d(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a: np.ndarray, offset_elems: int = 0):
    return ctypes.cast(a.ctypes.data + offset_elems * a.itemsize, _dp)


def scratch_row_len(n_in: int, n_hid: int, lib=None) -> int:
    lib = lib or load_oracle()
    return int(lib.oracle_scratch_row_len(n_in, n_hid))


def _row_chunks(B: int, threads: int):
    threads = max(1, min(threads, B))
    bounds = np.linspace(0, B, threads + 1).astype(int)
    return [(int(bounds[t]), int(bounds[t + 1])) for t in range(threads) if bounds[t + 1] > bounds[t]]


def cfc_forward(w_in, w_rec, b, w_tau, x, h0, dt, threads: int = 1, lib=None,
                cell: str = "gated") -> np.ndarray:
    """h_seq [B, K, H] in float64."""
    lib = lib or load_oracle()
    w_in, w_rec, b, w_tau, x, h0 = map(_d, (w_in, w_rec, b, w_tau, x, h0))
    B, K, n_in = x.shape
    H = w_rec.shape[0]
    h_seq = np.empty((B, K, H), dtype=np.float64)

    def run(r0, r1):
        rc = lib.oracle_cfc_forward(r1 - r0, K, n_in, H, float(dt), _ptr(w_in), _ptr(w_rec),
                                    _ptr(b), _ptr(w_tau), _ptr(x, r0 * K * n_in),
                                    _ptr(h0, r0 * H), _ptr(h_seq, r0 * K * H), CELLS[cell])
        if rc != 0:
            raise ValueError("oracle_cfc_forward rejected its arguments")

    _run_rows(run, B, threads)
    return h_seq


def cfc_backward(w_in, w_rec, b, w_tau, x, h0, h_seq, y, dt, threads: int = 1,
                 lib=None, scratch: Optional[np.ndarray] = None, cell: str = "gated"):
    """(scratch [B, N] float64, loss [B] float64).  ``scratch`` may be a
    preallocated (possibly poisoned) float64 buffer; the oracle zeroes it."""
    lib = lib or load_oracle()
    w_in, w_rec, b, w_tau, x, h0, h_seq, y = map(_d, (w_in, w_rec, b, w_tau, x, h0, h_seq, y))
    B, K, n_in = x.shape
    H = w_rec.shape[0]
    N = scratch_row_len(n_in, H, lib)
    if scratch is None:
        scratch = np.empty((B, N), dtype=np.float64)
    assert scratch.shape == (B, N) and scratch.dtype == np.float64 and scratch.flags.c_contiguous
    loss = np.empty(B, dtype=np.float64)

    def run(r0, r1):
        rc = lib.oracle_cfc_backward_inputs(r1 - r0, K, n_in, H, float(dt), _ptr(w_in), _ptr(w_rec),
                                            _ptr(b), _ptr(w_tau), _ptr(x, r0 * K * n_in),
                                            _ptr(h0, r0 * H), _ptr(h_seq, r0 * K * H), _ptr(y, r0 * H),
                                            _ptr(scratch, r0 * N), _ptr(loss, r0), None, None, CELLS[cell])
        if rc != 0:
            raise ValueError("oracle_cfc_backward_inputs rejected its arguments")

    _run_rows(run, B, threads)
    return scratch, loss


def cfc_backward_inputs(w_in, w_rec, b, w_tau, x, h0, h_seq, y, dt, threads: int = 1, lib=None,
                        cell: str = "gated"):
    """(scratch [B, N], loss [B], grad_x [B, K, n_in], grad_h0 [B, H]), float64:
    the backward plus the gradients with respect to x and h0."""
    lib = lib or load_oracle()
    w_in, w_rec, b, w_tau, x, h0, h_seq, y = map(_d, (w_in, w_rec, b, w_tau, x, h0, h_seq, y))
    B, K, n_in = x.shape
    H = w_rec.shape[0]
    N = scratch_row_len(n_in, H, lib)
    scratch = np.empty((B, N), dtype=np.float64)
    loss = np.empty(B, dtype=np.float64)
    grad_x = np.empty((B, K, n_in), dtype=np.float64)
    grad_h0 = np.empty((B, H), dtype=np.float64)

    def run(r0, r1):
        rc = lib.oracle_cfc_backward_inputs(
            r1 - r0, K, n_in, H, float(dt), _ptr(w_in), _ptr(w_rec), _ptr(b), _ptr(w_tau),
            _ptr(x, r0 * K * n_in), _ptr(h0, r0 * H), _ptr(h_seq, r0 * K * H), _ptr(y, r0 * H),
            _ptr(scratch, r0 * N), _ptr(loss, r0), _ptr(grad_x, r0 * K * n_in), _ptr(grad_h0, r0 * H),
            CELLS[cell])
        if rc != 0:
            raise ValueError("oracle_cfc_backward_inputs rejected its arguments")

    _run_rows(run, B, threads)
    return scratch, loss, grad_x, grad_h0


def reduce_axis0(per_batch, lib=None) -> np.ndarray:
    lib = lib or load_oracle()
    a = _d(per_batch)
    B, N = a.shape
    out = np.empty(N, dtype=np.float64)
    if lib.oracle_reduce_axis0(B, N, _ptr(a), _ptr(out)) != 0:
        raise ValueError("oracle_reduce_axis0 rejected its arguments")
    return out


def reduce_axis0_f32(per_batch_f32, lib=None) -> np.ndarray:
    """Column sums of a float32 matrix, each term widened to float64."""
    lib = lib or load_oracle()
    a = np.ascontiguousarray(per_batch_f32, dtype=np.float32)
    B, N = a.shape
    out = np.empty(N, dtype=np.float64)
    if lib.oracle_reduce_axis0_f32(B, N, ctypes.cast(a.ctypes.data, _fp), _ptr(out)) != 0:
        raise ValueError("oracle_reduce_axis0_f32 rejected its arguments")
    return out


def cfc_step(inp, threads: int = 1, lib=None, keep_scratch: bool = True,
             row_block: int = 256, input_grads: bool = False):
    """One whole step over a workload's inputs: forward, backward, reduce.

    Returns dict(h_seq, scratch (or None), loss, out), all float64, plus
    grad_x and grad_h0 with ``input_grads``.  With ``keep_scratch=False`` rows
    are processed in blocks and only the column sum (still b ascending) is
    kept, so memory stays O(row_block * N).
    """
    lib = lib or load_oracle()
    cell = getattr(inp, "cell", "gated")
    h_seq = cfc_forward(inp.w_in, inp.w_rec, inp.b, inp.w_tau, inp.x, inp.h0, inp.dt,
                        threads=threads, lib=lib, cell=cell)
    B = inp.x.shape[0]
    if input_grads:
        scratch, loss, gx, gh = cfc_backward_inputs(inp.w_in, inp.w_rec, inp.b, inp.w_tau, inp.x, inp.h0,
                                                    h_seq, inp.y, inp.dt, threads=threads, lib=lib, cell=cell)
        out = reduce_axis0(scratch, lib=lib)
        return dict(h_seq=h_seq, scratch=scratch, loss=loss, out=out, grad_x=gx, grad_h0=gh)
    if keep_scratch:
        scratch, loss = cfc_backward(inp.w_in, inp.w_rec, inp.b, inp.w_tau, inp.x, inp.h0,
                                     h_seq, inp.y, inp.dt, threads=threads, lib=lib, cell=cell)
        out = reduce_axis0(scratch, lib=lib)
        return dict(h_seq=h_seq, scratch=scratch, loss=loss, out=out)
    N = scratch_row_len(inp.x.shape[2], inp.w_rec.shape[0], lib)
    out = np.zeros(N, dtype=np.float64)
    loss = np.empty(B, dtype=np.float64)
    for r0 in range(0, B, row_block):
        r1 = min(B, r0 + row_block)
        s, l = cfc_backward(inp.w_in, inp.w_rec, inp.b, inp.w_tau, inp.x[r0:r1], inp.h0[r0:r1],
                            h_seq[r0:r1], inp.y[r0:r1], inp.dt, threads=threads, lib=lib, cell=cell)
        loss[r0:r1] = l
        for r in range(r1 - r0):       # b ascending, one row at a time
            out += s[r]
    return dict(h_seq=h_seq, scratch=None, loss=loss, out=out)


def _run_rows(fn, B: int, threads: int):
    chunks = _row_chunks(B, threads) if B > 0 else []
    if len(chunks) <= 1:
        for r0, r1 in chunks:
            fn(r0, r1)
        return
    with ThreadPoolExecutor(max_workers=len(chunks)) as ex:
        for f in [ex.submit(fn, r0, r1) for r0, r1 in chunks]:
            f.result()

"""Shared helpers for the GPU parity tests: upload seeded inputs, run the HIP
path through the C ABI, and compare with the float64 oracle element by element.

Tolerance rule (per element, the approx::relative_eq convention of the pages'
B=1 oracle test in the "K-loop Parallelization Implementation Plan", Task 6,
at the bar this library is held to):  pass iff
    |g - r| <= 1e-5   or   |g - r| <= 1e-4 * max(|g|, |r|).
"""
from __future__ import annotations

import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

RTOL = 1e-4
ATOL = 1e-5


def oracle_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def close_mask(got, want, rtol=RTOL, atol=ATOL):
    g = np.asarray(got, dtype=np.float64)
    r = np.asarray(want, dtype=np.float64)
    d = np.abs(g - r)
    return (d <= atol) | (d <= rtol * np.maximum(np.abs(g), np.abs(r)))


def assert_close(got, want, what: str, rtol=RTOL, atol=ATOL):
    ok = close_mask(got, want, rtol, atol)
    if not ok.all():
        g = np.asarray(got, dtype=np.float64).ravel()
        r = np.asarray(want, dtype=np.float64).ravel()
        bad = np.flatnonzero(~ok.ravel())
        d = np.abs(g - r)
        raise AssertionError(
            f"{what}: {bad.size} of {ok.size} elements outside |d|<={atol} or rel<={rtol}; "
            f"first bad index {bad[0]} got {g[bad[0]]!r} want {r[bad[0]]!r}; "
            f"max abs err {d.max():.3e}")
    return float(np.max(np.abs(np.asarray(got, np.float64) - np.asarray(want, np.float64)))) \
        if np.size(got) else 0.0


def to_dev(inp, device="cuda"):
    import torch
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)
    return dict(w_in=t(inp.w_in), w_rec=t(inp.w_rec), b=t(inp.b), w_tau=t(inp.w_tau),
                x=t(inp.x), h0=t(inp.h0), y=t(inp.y), dt=float(inp.dt))


def gpu_step(d, scratch=None, out=None, accumulate=False):
    """forward + backward + reduce on the current stream; returns device tensors."""
    import cfc_recurrent_cell_amd as C
    h_seq = C.cfc_forward(d["w_in"], d["w_rec"], d["b"], d["w_tau"], d["x"], d["h0"], d["dt"])
    scratch, loss = C.cfc_backward(d["w_in"], d["w_rec"], d["b"], d["w_tau"], d["x"], d["h0"],
                                   h_seq, d["y"], d["dt"], scratch=scratch, accumulate=accumulate)
    out = C.reduce_axis0(scratch, out=out)
    return h_seq, scratch, loss, out


def host(t):
    import torch
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def say(msg: str):
    print(msg, flush=True)

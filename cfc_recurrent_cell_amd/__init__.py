"""cfc_recurrent_cell_amd -- batched CfC cell K-loop on AMD MI355X (gfx950).

Thin Python layer over the C ABI in ``include/cfc.h``: it checks tensor
shapes, dtypes and devices, takes device pointers from torch tensors and the
current torch stream, and calls the HIP library.  PyTorch provides device
memory and streams only; every step of the computation runs in the library's
kernels.  Importing works without a GPU; calling needs the built library
(``python -m cfc_recurrent_cell_amd.build``) and raises if it is missing.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Tuple

from ._lib import (  # noqa: F401
    CELLS, CFC_CELL_GATED, CFC_CELL_TAU_DECAY, CFC_ACCUMULATE, CFC_ERR_DIM, CFC_ERR_DT, CFC_ERR_HIP, CFC_ERR_NULL, CFC_ERR_OVERLAP,
    CFC_ERR_UNSUPPORTED, CFC_OK, CFC_OVERWRITE, CfcError, CfcParams, LIB_PATH, _check,
    declared_symbols, load_library, status_string,
)

__all__ = ["cfc_forward", "cfc_backward", "cfc_backward_window", "cfc_backward_windows",
           "cfc_backward_workspace", "cfc_forward_backward_workspace", "cfc_forward_backward", "reduce_axis0", "reduce_axis0_noalloc",
           "reduce_axis0_split_workspace", "cfc_scratch_row_len", "CfcError", "load_library"]


def cfc_scratch_row_len(n_in: int, n_hid: int) -> int:
    """N = n_hid * (n_in + n_hid + 2); -1 for invalid dimensions."""
    return int(load_library().cfc_scratch_row_len(n_in, n_hid))


def _dev_f32(t, name, shape=None):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous float32 tensor on a GPU "
                         f"(got {t.dtype}, {t.device}, contiguous={t.is_contiguous()})")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


def _stream(device, stream):
    import torch
    s = torch.cuda.current_stream(device) if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _params(w_in, w_rec, b, w_tau, cell="gated"):
    if cell not in CELLS:
        raise ValueError(f"cell must be one of {sorted(CELLS)}, got {cell!r}")
    H, n_in = w_in.shape
    _dev_f32(w_in, "w_in", (H, n_in))
    _dev_f32(w_rec, "w_rec", (H, H))
    _dev_f32(b, "b", (H,))
    _dev_f32(w_tau, "w_tau", (H,))
    return CfcParams(w_in.data_ptr(), w_rec.data_ptr(), b.data_ptr(), w_tau.data_ptr(), n_in, H, CELLS[cell])


def cfc_forward(w_in, w_rec, b, w_tau, x, h0, dt: float, h_seq=None, stream=None, cell: str = "gated"):
    """h_seq [B, K, H] = forward K-loop of the cell (see include/cfc.h);
    ``cell`` is "gated" or "tau_decay" (w_tau then holds tau)."""
    import torch
    lib = load_library()
    p = _params(w_in, w_rec, b, w_tau, cell)
    B, K, _ = x.shape
    _dev_f32(x, "x", (B, K, p.n_in))
    _dev_f32(h0, "h0", (B, p.n_hid))
    if h_seq is None:
        h_seq = torch.empty((B, K, p.n_hid), dtype=torch.float32, device=x.device)
    _dev_f32(h_seq, "h_seq", (B, K, p.n_hid))
    _check("cfc_forward", lib.cfc_forward(ctypes.byref(p), x.data_ptr(), h0.data_ptr(),
                                          float(dt), B, K, h_seq.data_ptr(),
                                          _stream(x.device, stream)))
    return h_seq


def _input_grad_buffers(x, p, grad_x, grad_h0, input_grads):
    """Allocate (or check) the optional dL/dx [B, K, n_in] and dL/dh0 [B, H]."""
    import torch
    B, K, _ = x.shape
    if input_grads and grad_x is None:
        grad_x = torch.empty((B, K, p.n_in), dtype=torch.float32, device=x.device)
    if input_grads and grad_h0 is None:
        grad_h0 = torch.empty((B, p.n_hid), dtype=torch.float32, device=x.device)
    if grad_x is not None:
        _dev_f32(grad_x, "grad_x", (B, K, p.n_in))
    if grad_h0 is not None:
        _dev_f32(grad_h0, "grad_h0", (B, p.n_hid))
    return grad_x, grad_h0


def _workspace_arg(workspace):
    if workspace is None:
        return None, 0
    if workspace.device.type != "cuda" or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the GPU")
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


def _accumulate_workspace(x, p, K, accumulate, workspace, one_call=False):
    """The workspace accumulate mode needs at widths above 128 (K <= 20), allocated here when the
    caller passed none: without it that mode runs the general one-row-per-workgroup backward,
    about 8x slower at B=8192, K=8, 256/256.  The one-call entry gets its own size, which also
    holds its float64 weight copy at 256 x 256."""
    import torch
    if workspace is not None or not accumulate:
        return workspace
    size = cfc_forward_backward_workspace if one_call else cfc_backward_workspace
    need = size(x.shape[0], K, p.n_in, p.n_hid, accumulate=True)
    return torch.empty((need,), dtype=torch.uint8, device=x.device) if need > 0 else None


def cfc_backward_workspace(B: int, Kw: int, n_in: int, n_hid: int, accumulate: bool = True) -> int:
    """Bytes of workspace cfc_backward_window_ws needs for a window of Kw
    steps (0: the window's kernel uses none)."""
    n = int(load_library().cfc_backward_workspace(B, Kw, n_in, n_hid,
                                                   CFC_ACCUMULATE if accumulate else CFC_OVERWRITE))
    if n < 0:
        raise ValueError(f"invalid backward size B={B} Kw={Kw} n_in={n_in} n_hid={n_hid}")
    return n


def cfc_forward_backward_workspace(B: int, K: int, n_in: int, n_hid: int, accumulate: bool = True) -> int:
    """Bytes of workspace cfc_forward_backward_ws runs best with: the backward's
    size, plus its float64 weight copy at 256 x 256 with K <= 8."""
    n = int(load_library().cfc_forward_backward_workspace(B, K, n_in, n_hid,
                                                          CFC_ACCUMULATE if accumulate else CFC_OVERWRITE))
    if n < 0:
        raise ValueError(f"invalid size B={B} K={K} n_in={n_in} n_hid={n_hid}")
    return n


def cfc_backward(w_in, w_rec, b, w_tau, x, h0, h_seq, y, dt: float, scratch=None,
                 loss=None, accumulate: bool = False, want_loss: bool = True,
                 input_grads: bool = False, grad_x=None, grad_h0=None,
                 stream=None, cell: str = "gated", workspace=None) -> Tuple[object, ...]:
    """(scratch [B, N], loss [B] or None): per-row parameter gradients of
    L_b = 1/2 |h_K - y_b|^2 (see include/cfc.h for the row layout).  With
    ``input_grads`` (or explicit ``grad_x`` / ``grad_h0`` buffers) it returns
    (scratch, loss, grad_x [B, K, n_in], grad_h0 [B, H]) instead.  Accumulate
    mode at widths above 128 with K <= 20 runs the 16-row kernel through
    cfc_backward_window_ws with a device ``workspace`` of
    cfc_backward_workspace bytes, allocated here unless given."""
    import torch
    lib = load_library()
    p = _params(w_in, w_rec, b, w_tau, cell)
    B, K, _ = x.shape
    N = cfc_scratch_row_len(p.n_in, p.n_hid)
    _dev_f32(x, "x", (B, K, p.n_in))
    _dev_f32(h0, "h0", (B, p.n_hid))
    _dev_f32(h_seq, "h_seq", (B, K, p.n_hid))
    _dev_f32(y, "y", (B, p.n_hid))
    if scratch is None:
        scratch = torch.empty((B, N), dtype=torch.float32, device=x.device)
    _dev_f32(scratch, "scratch", (B, N))
    if loss is None and want_loss:
        loss = torch.empty((B,), dtype=torch.float32, device=x.device)
    if loss is not None:
        _dev_f32(loss, "loss", (B,))
    want_inputs = input_grads or grad_x is not None or grad_h0 is not None
    grad_x, grad_h0 = _input_grad_buffers(x, p, grad_x, grad_h0, input_grads)
    flags = CFC_ACCUMULATE if accumulate else CFC_OVERWRITE
    ptr = lambda t: t.data_ptr() if t is not None else None
    workspace = _accumulate_workspace(x, p, K, accumulate, workspace)
    if workspace is not None:
        ws_ptr, ws_bytes = _workspace_arg(workspace)
        _check("cfc_backward_window_ws", lib.cfc_backward_window_ws(
            ctypes.byref(p), x.data_ptr(), h0.data_ptr(), h_seq.data_ptr(), y.data_ptr(), None, float(dt),
            B, K, 0, K, scratch.data_ptr(), ptr(loss), ptr(grad_x), ptr(grad_h0), flags, ws_ptr, ws_bytes,
            _stream(x.device, stream)))
    else:
        _check("cfc_backward", lib.cfc_backward(
            ctypes.byref(p), x.data_ptr(), h0.data_ptr(), h_seq.data_ptr(), y.data_ptr(), float(dt),
            B, K, scratch.data_ptr(), ptr(loss), ptr(grad_x), ptr(grad_h0), flags,
            _stream(x.device, stream)))
    if want_inputs:
        return scratch, loss, grad_x, grad_h0
    return scratch, loss


def cfc_backward_window(w_in, w_rec, b, w_tau, x, h0, h_seq, dt: float, k_begin: int, k_end: int, scratch,
                        y=None, delta_in=None, delta_out=None, loss=None, grad_x=None,
                        accumulate: bool = False, stream=None, cell: str = "gated", workspace=None):
    """Backward over steps [k_begin, k_end) of the forward that produced
    h_seq (see include/cfc.h): dL/dh_k_end comes in as ``delta_in`` (or, when
    None, from the loss seed h_K - y), dL/dh_k_begin goes out in ``delta_out``
    (may be ``delta_in`` itself), the window's parameter gradient goes into
    ``scratch`` (overwritten, or added with ``accumulate``).  With a device
    ``workspace`` it calls cfc_backward_window_ws.  Returns
    (scratch, loss, grad_x, delta_out)."""
    lib = load_library()
    p = _params(w_in, w_rec, b, w_tau, cell)
    B, K, _ = x.shape
    N = cfc_scratch_row_len(p.n_in, p.n_hid)
    _dev_f32(x, "x", (B, K, p.n_in))
    _dev_f32(h0, "h0", (B, p.n_hid))
    _dev_f32(h_seq, "h_seq", (B, K, p.n_hid))
    _dev_f32(scratch, "scratch", (B, N))
    for t, name, shape in ((y, "y", (B, p.n_hid)), (delta_in, "delta_in", (B, p.n_hid)),
                           (delta_out, "delta_out", (B, p.n_hid)), (loss, "loss", (B,)),
                           (grad_x, "grad_x", (B, K, p.n_in))):
        if t is not None:
            _dev_f32(t, name, shape)
    ptr = lambda t: t.data_ptr() if t is not None else None
    flags = CFC_ACCUMULATE if accumulate else CFC_OVERWRITE
    if workspace is not None:
        ws_ptr, ws_bytes = _workspace_arg(workspace)
        _check("cfc_backward_window_ws", lib.cfc_backward_window_ws(
            ctypes.byref(p), x.data_ptr(), h0.data_ptr(), h_seq.data_ptr(), ptr(y), ptr(delta_in), float(dt), B,
            K, int(k_begin), int(k_end), scratch.data_ptr(), ptr(loss), ptr(grad_x), ptr(delta_out), flags, ws_ptr,
            ws_bytes, _stream(x.device, stream)))
    else:
        _check("cfc_backward_window", lib.cfc_backward_window(
            ctypes.byref(p), x.data_ptr(), h0.data_ptr(), h_seq.data_ptr(), ptr(y), ptr(delta_in), float(dt), B,
            K, int(k_begin), int(k_end), scratch.data_ptr(), ptr(loss), ptr(grad_x), ptr(delta_out), flags,
            _stream(x.device, stream)))
    return scratch, loss, grad_x, delta_out


def cfc_backward_windows(w_in, w_rec, b, w_tau, x, h0, h_seq, y, dt: float, window: int, scratch=None,
                         loss=None, grad_x=None, grad_h0=None, stream=None, cell: str = "gated",
                         workspace=None):
    """The whole backward as windows of ``window`` steps, from the last to the
    first: the last window is seeded from y and overwrites the scratch, each
    earlier one takes the carried dL/dh and accumulates.  For K beyond the
    one-call backward's on-chip limit.  The accumulating windows get a device
    workspace (allocated here unless given; none where their kernel needs
    none).  Returns (scratch, loss, grad_x, grad_h0) with grad_h0 = dL/dh_0
    (allocated here if not given)."""
    import torch
    B, K, _ = x.shape
    if window < 1:
        raise ValueError("window must be >= 1")
    H = w_rec.shape[0]
    if workspace is None and K > window:
        need = cfc_backward_workspace(B, window, w_in.shape[1], H, accumulate=True)
        if need > 0:
            workspace = torch.empty((need,), dtype=torch.uint8, device=x.device)
    if scratch is None:
        scratch = torch.empty((B, cfc_scratch_row_len(w_in.shape[1], H)), dtype=torch.float32, device=x.device)
    if loss is None:
        loss = torch.empty((B,), dtype=torch.float32, device=x.device)
    delta = grad_h0 if grad_h0 is not None else torch.empty((B, H), dtype=torch.float32, device=x.device)
    k_end = K
    while k_end > 0:
        k_begin = max(0, k_end - window)
        seeded = k_end == K
        cfc_backward_window(w_in, w_rec, b, w_tau, x, h0, h_seq, dt, k_begin, k_end, scratch,
                            y=y if seeded else None, delta_in=None if seeded else delta, delta_out=delta,
                            loss=loss if seeded else None, grad_x=grad_x, accumulate=not seeded, stream=stream,
                            cell=cell, workspace=workspace)
        k_end = k_begin
    return scratch, loss, grad_x, delta


def cfc_forward_backward(w_in, w_rec, b, w_tau, x, h0, y, dt: float, h_seq=None, scratch=None,
                         loss=None, accumulate: bool = False, want_loss: bool = True,
                         input_grads: bool = False, grad_x=None, grad_h0=None,
                         stream=None, cell: str = "gated", workspace=None) -> Tuple[object, ...]:
    """(h_seq [B, K, H], scratch [B, N], loss [B] or None): the forward and the
    backward of the same inputs in one library call (see include/cfc.h).  With
    ``input_grads`` (or explicit buffers) grad_x and grad_h0 are appended.
    Accumulate mode at widths above 128 with K <= 20 runs the 16-row backward
    through cfc_forward_backward_ws with a device ``workspace`` of
    cfc_forward_backward_workspace bytes (at least cfc_backward_workspace),
    allocated here unless given."""
    import torch
    lib = load_library()
    p = _params(w_in, w_rec, b, w_tau, cell)
    B, K, _ = x.shape
    N = cfc_scratch_row_len(p.n_in, p.n_hid)
    _dev_f32(x, "x", (B, K, p.n_in))
    _dev_f32(h0, "h0", (B, p.n_hid))
    _dev_f32(y, "y", (B, p.n_hid))
    if h_seq is None:
        h_seq = torch.empty((B, K, p.n_hid), dtype=torch.float32, device=x.device)
    _dev_f32(h_seq, "h_seq", (B, K, p.n_hid))
    if scratch is None:
        scratch = torch.empty((B, N), dtype=torch.float32, device=x.device)
    _dev_f32(scratch, "scratch", (B, N))
    if loss is None and want_loss:
        loss = torch.empty((B,), dtype=torch.float32, device=x.device)
    if loss is not None:
        _dev_f32(loss, "loss", (B,))
    want_inputs = input_grads or grad_x is not None or grad_h0 is not None
    grad_x, grad_h0 = _input_grad_buffers(x, p, grad_x, grad_h0, input_grads)
    flags = CFC_ACCUMULATE if accumulate else CFC_OVERWRITE
    ptr = lambda t: t.data_ptr() if t is not None else None
    workspace = _accumulate_workspace(x, p, K, accumulate, workspace, one_call=True)
    if workspace is not None:
        ws_ptr, ws_bytes = _workspace_arg(workspace)
        _check("cfc_forward_backward_ws", lib.cfc_forward_backward_ws(
            ctypes.byref(p), x.data_ptr(), h0.data_ptr(), y.data_ptr(), float(dt), B, K,
            h_seq.data_ptr(), scratch.data_ptr(), ptr(loss), ptr(grad_x), ptr(grad_h0), flags, ws_ptr, ws_bytes,
            _stream(x.device, stream)))
    else:
        _check("cfc_forward_backward", lib.cfc_forward_backward(
            ctypes.byref(p), x.data_ptr(), h0.data_ptr(), y.data_ptr(), float(dt), B, K,
            h_seq.data_ptr(), scratch.data_ptr(), ptr(loss), ptr(grad_x), ptr(grad_h0), flags,
            _stream(x.device, stream)))
    if want_inputs:
        return h_seq, scratch, loss, grad_x, grad_h0
    return h_seq, scratch, loss


def reduce_axis0(per_batch, out=None, stream=None, leading_axes: int = 1, split: bool = False,
                 workspace=None):
    """Column sums over the leading axis (overwrites ``out``).

    ``per_batch`` is contiguous float32 on the GPU.  Its first ``leading_axes``
    dimensions are merged into the reduced axis B and the rest into the
    column axis N -- e.g. a [B, heads, E, H, H] scratch reduced over batch and
    heads is reduce_axis0(t, leading_axes=2) with B = B*heads and N = E*H*H
    (sizing N from the wrong axes reads past the buffer; here both come from
    the tensor's shape).  ``out`` gets shape per_batch.shape[leading_axes:].
    ``split=True`` uses reduce_axis0_split (narrow rows over a long leading
    axis); its workspace is allocated here unless given as a uint8 tensor."""
    import math
    import torch
    lib = load_library()
    if not 1 <= leading_axes <= per_batch.dim():
        raise ValueError(f"leading_axes must be in [1, {per_batch.dim()}], got {leading_axes}")
    _dev_f32(per_batch, "per_batch")
    lead, tail = tuple(per_batch.shape[:leading_axes]), tuple(per_batch.shape[leading_axes:])
    B, N = math.prod(lead), math.prod(tail)
    if out is None:
        out = torch.empty(tail, dtype=torch.float32, device=per_batch.device)
    _dev_f32(out, "out", tail)
    s = _stream(per_batch.device, stream)
    if not split:
        _check("reduce_axis0", lib.reduce_axis0(per_batch.data_ptr(), B, N, out.data_ptr(), s))
        return out
    need = int(lib.reduce_axis0_split_workspace(B, N))
    if need < 0:
        raise ValueError(f"invalid reduce size B={B} N={N}")
    if workspace is None and need > 0:
        workspace = torch.empty((need,), dtype=torch.uint8, device=per_batch.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("reduce_axis0_split", lib.reduce_axis0_split(per_batch.data_ptr(), B, N, out.data_ptr(), ws_ptr,
                                                        ws_bytes, s))
    return out


def reduce_axis0_noalloc(per_batch, out, stream=None, leading_axes: int = 1):
    """reduce_axis0_split_noalloc: the split column sum with its partials in
    the library's static device array, for callers that cannot allocate
    (graph capture, serving loops).  ``out`` must be given; neither the
    binding nor the library allocates.  Calls that overlap on one GPU share
    that array and must be serialised (one stream)."""
    import math
    lib = load_library()
    if not 1 <= leading_axes <= per_batch.dim():
        raise ValueError(f"leading_axes must be in [1, {per_batch.dim()}], got {leading_axes}")
    _dev_f32(per_batch, "per_batch")
    tail = tuple(per_batch.shape[leading_axes:])
    B, N = math.prod(per_batch.shape[:leading_axes]), math.prod(tail)
    _dev_f32(out, "out", tail)
    _check("reduce_axis0_split_noalloc", lib.reduce_axis0_split_noalloc(per_batch.data_ptr(), B, N, out.data_ptr(),
                                                                        _stream(per_batch.device, stream)))
    return out


def reduce_axis0_split_workspace(B: int, N: int) -> int:
    """Bytes of workspace reduce_axis0_split needs for [B, N] (0: none)."""
    return int(load_library().reduce_axis0_split_workspace(B, N))

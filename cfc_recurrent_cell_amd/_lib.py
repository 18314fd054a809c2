"""ctypes binding of libcfc_amd.so: argument marshalling only.

Every step of the path runs in the HIP library.  If the library is missing
the import of the functions below raises; there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os
import re

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libcfc_amd.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "cfc.h")

CFC_OK = 0
CFC_ERR_NULL = 1
CFC_ERR_DIM = 2
CFC_ERR_DT = 3
CFC_ERR_UNSUPPORTED = 4
CFC_ERR_OVERLAP = 5
CFC_ERR_HIP = 6
CFC_OVERWRITE = 0
CFC_ACCUMULATE = 1


CFC_CELL_GATED = 0
CFC_CELL_TAU_DECAY = 1
CELLS = {"gated": CFC_CELL_GATED, "tau_decay": CFC_CELL_TAU_DECAY}


class CfcParams(ctypes.Structure):
    _fields_ = [("w_in", ctypes.c_void_p), ("w_rec", ctypes.c_void_p), ("b", ctypes.c_void_p),
                ("w_tau", ctypes.c_void_p), ("n_in", ctypes.c_int), ("n_hid", ctypes.c_int),
                ("cell", ctypes.c_int)]


class CfcError(RuntimeError):
    def __init__(self, fn: str, code: int, text: str):
        super().__init__(f"{fn} failed with status {code}: {text}")
        self.code = code


_lib = None


def load_library(path: str = LIB_PATH):
    """Load the built HIP library; raise loudly if it is absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(
            f"libcfc_amd.so not found at {path}; build it with "
            "`python -m cfc_recurrent_cell_amd.build` (hipcc, gfx950). There is no CPU fallback.")
    lib = ctypes.CDLL(path)
    vp, i, ll, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_longlong, ctypes.c_float
    lib.cfc_scratch_row_len.restype = ll
    lib.cfc_scratch_row_len.argtypes = [i, i]
    lib.cfc_forward.restype = i
    lib.cfc_forward.argtypes = [ctypes.POINTER(CfcParams), vp, vp, f, i, i, vp, vp]
    lib.cfc_backward.restype = i
    lib.cfc_backward.argtypes = [ctypes.POINTER(CfcParams), vp, vp, vp, vp, f, i, i, vp, vp, vp, vp, i, vp]
    lib.cfc_backward_window.restype = i
    lib.cfc_backward_window.argtypes = [ctypes.POINTER(CfcParams), vp, vp, vp, vp, vp, f, i, i, i, i, vp, vp, vp,
                                        vp, i, vp]
    lib.cfc_backward_workspace.restype = ll
    lib.cfc_backward_workspace.argtypes = [i, i, i, i, i]
    lib.cfc_forward_backward_workspace.restype = ll
    lib.cfc_forward_backward_workspace.argtypes = [i, i, i, i, i]
    lib.cfc_backward_window_ws.restype = i
    lib.cfc_backward_window_ws.argtypes = [ctypes.POINTER(CfcParams), vp, vp, vp, vp, vp, f, i, i, i, i, vp, vp,
                                           vp, vp, i, vp, ll, vp]
    lib.cfc_forward_backward.restype = i
    lib.cfc_forward_backward.argtypes = [ctypes.POINTER(CfcParams), vp, vp, vp, f, i, i, vp, vp, vp, vp, vp,
                                         i, vp]
    lib.cfc_forward_backward_ws.restype = i
    lib.cfc_forward_backward_ws.argtypes = [ctypes.POINTER(CfcParams), vp, vp, vp, f, i, i, vp, vp, vp, vp, vp,
                                            i, vp, ll, vp]
    lib.reduce_axis0.restype = i
    lib.reduce_axis0.argtypes = [vp, ll, ll, vp, vp]
    lib.reduce_axis0_split_workspace.restype = ll
    lib.reduce_axis0_split_workspace.argtypes = [ll, ll]
    lib.reduce_axis0_split.restype = i
    lib.reduce_axis0_split.argtypes = [vp, ll, ll, vp, vp, ll, vp]
    lib.reduce_axis0_split_noalloc.restype = i
    lib.reduce_axis0_split_noalloc.argtypes = [vp, ll, ll, vp, vp]
    lib.cfc_status_string.restype = ctypes.c_char_p
    lib.cfc_status_string.argtypes = [i]
    _lib = lib
    return lib


def declared_symbols(header: str = HEADER):
    """Names of the functions include/cfc.h declares."""
    with open(header) as fh:
        text = fh.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w \*]*?\b(\w+)\s*\(", text, flags=re.M)))


def status_string(code: int) -> str:
    return load_library().cfc_status_string(code).decode()


def _check(fn: str, code: int):
    if code != CFC_OK:
        raise CfcError(fn, code, status_string(code))
    return code

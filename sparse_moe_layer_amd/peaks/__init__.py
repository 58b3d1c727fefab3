"""ctypes binding of libmoe_peaks.so (include/moe_peaks.h): the peak-rate probes that the
benchmark quotes the layer's roofline fractions against.  Not part of the layer."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_peaks.so")
EXPORTS = ("moe_peak_read", "moe_peak_mfma")
_lib = None


def lib():
    """The loaded libmoe_peaks.so (raises if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
    try:   # share torch's HIP runtime
        import torch  # noqa: F401
    except ImportError:
        pass
    L = ctypes.CDLL(LIB_PATH)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32
    L.moe_peak_read.argtypes = [vp, sz, vp, sz, i32, vp]
    L.moe_peak_mfma.argtypes = [i32, i32, i32, vp, sz, ctypes.POINTER(ctypes.c_double), vp]
    for f in EXPORTS:
        getattr(L, f).restype = ctypes.c_int
    _lib = L
    return L


def check(status: int):
    if status != 0:
        raise RuntimeError(f"peak probe failed with status {status}")

"""Seeded synthetic inputs shared by the CPU oracle and the GPU path.

Holds parameter lists / buckets (``workloads``) and the counter-based value
generator in two byte-identical implementations: host C (``libsynth_host.so``)
and device HIP (``libsynth_dev.so``).  No reduction arithmetic lives here.
"""
import ctypes
import os

import numpy as np

from . import workloads  # noqa: F401
from .workloads import DT_BF16, DT_F32  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_host = None
_dev = None


def _load_host():
    global _host
    if _host is None:
        path = os.path.join(_HERE, "libsynth_host.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(path)
        lib.synth_fill_host.argtypes = [ctypes.c_int, ctypes.c_uint64, ctypes.c_uint64,
                                        ctypes.c_uint32, ctypes.c_uint32, ctypes.c_int64,
                                        ctypes.c_int64, ctypes.c_void_p]
        lib.synth_fill_host.restype = None
        lib.synth_gather_host.argtypes = [ctypes.c_int, ctypes.c_uint64, ctypes.c_uint64,
                                          ctypes.c_uint32, ctypes.c_uint32, ctypes.c_void_p,
                                          ctypes.c_int64, ctypes.c_void_p]
        lib.synth_gather_host.restype = None
        _host = lib
    return _host


def _load_dev():
    global _dev
    if _dev is None:
        path = os.path.join(_HERE, "libsynth_dev.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run __graft_entry__.build()")
        import torch  # noqa: F401  (torch's HIP runtime first, as for libdc)
        lib = ctypes.CDLL(path)
        lib.synth_fill_slab_device.argtypes = [ctypes.c_int, ctypes.c_uint64, ctypes.c_uint64,
                                               ctypes.c_uint32, ctypes.c_uint32, ctypes.c_int32,
                                               ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                                               ctypes.c_void_p]
        lib.synth_fill_slab_device.restype = ctypes.c_int
        lib.synth_fill_slab_device_at.argtypes = [ctypes.c_int, ctypes.c_uint64, ctypes.c_uint64,
                                                  ctypes.c_uint32, ctypes.c_uint32, ctypes.c_int32,
                                                  ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                                  ctypes.c_void_p, ctypes.c_void_p]
        lib.synth_fill_slab_device_at.restype = ctypes.c_int
        _dev = lib
    return _dev


def np_dtype(dtype: int):
    return np.uint16 if dtype == DT_BF16 else np.uint32


def fill_row(dtype: int, seed: int, stream: int, scale, col0: int, n: int) -> np.ndarray:
    """Host values of columns [col0, col0+n) of one rank row (raw bits)."""
    out = np.empty(n, dtype=np_dtype(dtype))
    C, E = scale
    _load_host().synth_fill_host(dtype, seed, stream, C, E, col0, n,
                                 out.ctypes.data_as(ctypes.c_void_p))
    return out


def fill_slab(dtype: int, seed: int, stream0: int, scale, rows: int, ld: int, ncols: int,
              out: np.ndarray = None) -> np.ndarray:
    """Host [rows, ld] slab; columns >= ncols are zero."""
    if out is None:
        out = np.zeros((rows, ld), dtype=np_dtype(dtype))
    for r in range(rows):
        out[r, :ncols] = fill_row(dtype, seed, stream0 + r, scale, 0, ncols)
    return out


def gather(dtype: int, seed: int, stream: int, scale, cols: np.ndarray) -> np.ndarray:
    """Host values of the listed columns of one rank row (raw bits)."""
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    out = np.empty(len(cols), dtype=np_dtype(dtype))
    C, E = scale
    _load_host().synth_gather_host(dtype, seed, stream, C, E,
                                   cols.ctypes.data_as(ctypes.c_void_p), len(cols),
                                   out.ctypes.data_as(ctypes.c_void_p))
    return out


def fill_slab_device(dtype: int, seed: int, stream0: int, scale, rows: int, ld: int,
                     ncols: int, ptr: int, hip_stream: int, col0: int = 0) -> None:
    """Fill a device [rows, ld] slab at `ptr` on `hip_stream` (raw handle):
    position j of row r holds column col0 + j of stream stream0 + r."""
    C, E = scale
    rc = _load_dev().synth_fill_slab_device_at(dtype, seed, stream0, C, E, rows, ld, ncols, col0,
                                               ctypes.c_void_p(ptr), ctypes.c_void_p(hip_stream))
    if rc != 0:
        raise RuntimeError(f"synth_fill_slab_device failed with code {rc}")

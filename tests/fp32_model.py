"""ctypes front end of tests/pins/fp32_model.c (test code).

The model reproduces, in IEEE binary32 on the CPU, the arithmetic contract
the library documents for its kernels (fixed sum-of-squares tree, correctly
rounded division and square root), so GPU results can be compared with it
bit for bit.  It is pinned against the binary64 oracle by the CPU tests.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "pins", "fp32_model.c")
LIBRARY = os.path.join(HERE, "pins", "libfp32model.so")
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
          "-fno-tree-vectorize"]

_lib = None


def build(force: bool = True) -> str:
    if force or not os.path.exists(LIBRARY) or (
            os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE)):
        tmp = LIBRARY + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", *CFLAGS, "-o", tmp, SOURCE, "-lm"], check=True)
        os.replace(tmp, LIBRARY)
    return LIBRARY


def lib():
    global _lib
    if _lib is None:
        build(force=False)
        L = ctypes.CDLL(LIBRARY)
        vp = ctypes.c_void_p
        L.model_add_rmsnorm.restype = ctypes.c_int
        L.model_add_rmsnorm.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_int64, ctypes.c_int64,
                                        ctypes.c_float]
        L.model_add_rmsnorm_quant.restype = ctypes.c_int
        L.model_add_rmsnorm_quant.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_int64,
                                              ctypes.c_int64, ctypes.c_float]
        L.model_add_rmsnorm_quant_fp8.restype = ctypes.c_int
        L.model_add_rmsnorm_quant_fp8.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_int64,
                                                  ctypes.c_int64, ctypes.c_float]
        L.model_e4m3_codes.restype = ctypes.c_int
        L.model_e4m3_codes.argtypes = [vp, vp, ctypes.c_int64]
        _lib = L
    return _lib


def _ptr(a):
    return a.ctypes.data if a is not None else None


def add_rmsnorm(x, residual, weight, eps=1e-6, want_sumsq=False):
    """(out, residual_out[, sum of squares per row]) of the fp32 model.
    residual None is plain RMSNorm; residual_out is then None."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    if residual is not None:
        residual = np.ascontiguousarray(residual, dtype=np.uint16)
    weight = np.ascontiguousarray(weight, dtype=np.uint16)
    n, h = x.shape
    out = np.empty_like(x)
    res = np.empty_like(x) if residual is not None else None
    ss = np.empty(n, dtype=np.float32) if want_sumsq else None
    rc = lib().model_add_rmsnorm(out.ctypes.data, _ptr(res), _ptr(ss), x.ctypes.data,
                                 _ptr(residual), weight.ctypes.data, n, h, ctypes.c_float(eps))
    if rc != 0:
        raise ValueError("fp32 model rejected its arguments")
    return (out, res, ss) if want_sumsq else (out, res)


def add_rmsnorm_quant(x, residual, weight, eps=1e-6):
    """(codes int8, scale fp32 per row, residual_out) of the fp32 model.
    residual None is plain RMSNorm; residual_out is then None."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    if residual is not None:
        residual = np.ascontiguousarray(residual, dtype=np.uint16)
    weight = np.ascontiguousarray(weight, dtype=np.uint16)
    n, h = x.shape
    q = np.empty(x.shape, dtype=np.int8)
    sc = np.empty(n, dtype=np.float32)
    res = np.empty_like(x) if residual is not None else None
    rc = lib().model_add_rmsnorm_quant(q.ctypes.data, sc.ctypes.data, _ptr(res), x.ctypes.data,
                                       _ptr(residual), weight.ctypes.data, n, h,
                                       ctypes.c_float(eps))
    if rc != 0:
        raise ValueError("fp32 model rejected its arguments")
    return q, sc, res


def add_rmsnorm_quant_fp8(x, residual, weight, eps=1e-6):
    """(E4M3 codes uint8, scale fp32 per row, residual_out) of the fp32 model.
    residual None is plain RMSNorm; residual_out is then None."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    if residual is not None:
        residual = np.ascontiguousarray(residual, dtype=np.uint16)
    weight = np.ascontiguousarray(weight, dtype=np.uint16)
    n, h = x.shape
    q = np.empty(x.shape, dtype=np.uint8)
    sc = np.empty(n, dtype=np.float32)
    res = np.empty_like(x) if residual is not None else None
    rc = lib().model_add_rmsnorm_quant_fp8(q.ctypes.data, sc.ctypes.data, _ptr(res),
                                           x.ctypes.data, _ptr(residual), weight.ctypes.data, n,
                                           h, ctypes.c_float(eps))
    if rc != 0:
        raise ValueError("fp32 model rejected its arguments")
    return q, sc, res


def e4m3_codes(v):
    """The model's E4M3 code of each binary32 value (|v| < 464)."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, dtype=np.uint8)
    lib().model_e4m3_codes(out.ctypes.data, v.ctypes.data, v.size)
    return out

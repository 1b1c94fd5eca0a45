"""ctypes front end of the fp64 CPU oracle (gemm_oracle.c) plus a library-matmul
evaluation of the same definition.

TEST INFRASTRUCTURE ONLY (see the package docstring). The definition followed
is the plain dense product C = A.B behind the pages' GEMM measurements
("GPU speed, without leaving Rust's safety model", section "Safety without a
visible tax"), with D = |A|.|B| as the tolerance scale.

Matrices are passed as numpy ``uint16`` arrays holding bf16 bit patterns.
Any positive numpy strides are honoured, so a column-major B is simply the
transpose view of a row-major N x K array.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
import sys

import numpy as np

from .numerics import bf16_to_f64

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gemm_oracle.c")
_SO = os.path.join(_HERE, "_gemm_oracle.so")
_lib = None


def lib_path() -> str:
    return _SO


def build(force: bool = True) -> str:
    """Compile gemm_oracle.c with gcc into oracle/_gemm_oracle.so.

    Portable flags only (no -march=native): the built library travels to
    machines with other CPUs.
    """
    global _lib
    if not force and os.path.exists(_SO) and os.path.getmtime(_SO) >= os.path.getmtime(_SRC):
        return _SO
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
           "-o", _SO + ".tmp", _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_SO + ".tmp", _SO)
    _lib = None
    return _SO


def open_library(path: str):
    """Load and configure a compiled oracle library (the default one, or a
    deliberately broken copy that a test builds to check that the pins fail)."""
    lib = ctypes.CDLL(path)
    i64, vp, dp = ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p
    lib.oracle_gemm_f64.argtypes = [vp, i64, i64, vp, i64, i64, i64, i64, i64,
                                    dp, dp, ctypes.c_int]
    lib.oracle_gemm_f64.restype = ctypes.c_int
    lib.oracle_gemm_f64_at.argtypes = [vp, i64, i64, vp, i64, i64, i64, vp, vp,
                                       i64, dp, dp, ctypes.c_int]
    lib.oracle_gemm_f64_at.restype = ctypes.c_int
    lib.oracle_max_threads.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        build()
    _lib = open_library(_SO)
    return _lib


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def _default_threads(threads):
    if threads is not None:
        return int(threads)
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _estrides(a: np.ndarray):
    if a.dtype != np.uint16:
        raise TypeError("bf16 operands are passed as uint16 bit patterns")
    if a.ndim != 2:
        raise ValueError("operands must be 2-D")
    s0, s1 = (st // a.itemsize for st in a.strides)
    if a.size and (s0 < 0 or s1 < 0):
        raise ValueError("negative strides are not supported")
    return s0, s1


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data) if a.size else None


def gemm(A: np.ndarray, B: np.ndarray, want_d: bool = True, threads=None, lib=None):
    """Full product by the fp64 triple loop. Returns (C, D or None)."""
    M, K = A.shape
    K2, N = B.shape
    if K2 != K:
        raise ValueError(f"inner dimensions differ: A is {A.shape}, B is {B.shape}")
    a_m, a_k = _estrides(A)
    b_k, b_n = _estrides(B)
    C = np.empty((M, N), np.float64)
    D = np.empty((M, N), np.float64) if want_d else None
    if C.size == 0:
        return C, D
    rc = (lib or _load()).oracle_gemm_f64(
        _ptr(A), a_m, a_k, _ptr(B), b_k, b_n, M, N, K,
        ctypes.c_void_p(C.ctypes.data),
        ctypes.c_void_p(D.ctypes.data) if D is not None else None,
        _default_threads(threads))
    if rc != 0:
        raise RuntimeError("oracle_gemm_f64 failed")
    return C, D


def gemm_at(A: np.ndarray, B: np.ndarray, ii, jj, threads=None, lib=None):
    """Selected elements C[ii[t], jj[t]] and D[ii[t], jj[t]], one at a time."""
    M, K = A.shape
    K2, N = B.shape
    if K2 != K:
        raise ValueError("inner dimensions differ")
    ii = np.ascontiguousarray(ii, dtype=np.int64)
    jj = np.ascontiguousarray(jj, dtype=np.int64)
    if ii.shape != jj.shape or ii.ndim != 1:
        raise ValueError("ii and jj must be 1-D and of equal length")
    if ii.size and (ii.min() < 0 or ii.max() >= M or jj.min() < 0 or jj.max() >= N):
        raise IndexError("sample index out of range")
    a_m, a_k = _estrides(A)
    b_k, b_n = _estrides(B)
    c = np.empty(ii.size, np.float64)
    d = np.empty(ii.size, np.float64)
    if ii.size == 0:
        return c, d
    rc = (lib or _load()).oracle_gemm_f64_at(
        _ptr(A), a_m, a_k, _ptr(B), b_k, b_n, K,
        ctypes.c_void_p(ii.ctypes.data), ctypes.c_void_p(jj.ctypes.data), ii.size,
        ctypes.c_void_p(c.ctypes.data), ctypes.c_void_p(d.ctypes.data),
        _default_threads(threads))
    if rc != 0:
        raise RuntimeError("oracle_gemm_f64_at failed")
    return c, d


def gemm_blas(A: np.ndarray, B: np.ndarray, want_d: bool = True):
    """The same definition, evaluated by numpy's fp64 matrix product.

    A library matmul sums in its own order, so this differs from the triple
    loop only by fp64 rounding (|error| <= K * 2^-53 * D); for integer-valued
    inputs every partial sum is an integer below 2^53 and both are exact.
    """
    A64 = bf16_to_f64(A)
    B64 = bf16_to_f64(B)
    C = A64 @ B64
    D = None
    if want_d:
        np.abs(A64, out=A64)
        np.abs(B64, out=B64)
        D = A64 @ B64
    return C, D


if __name__ == "__main__":  # pragma: no cover
    print(build(), file=sys.stderr)

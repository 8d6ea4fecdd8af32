"""CPU oracle for SGEMM: C = alpha * op(A) * op(B) + beta * C.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package. The GPU library and
its Python binding never import it, and the two share no code.

Definition followed: "Optimising fp32 GEMM on A100", section "What is GEMM?"
(C = alpha*(A x B) + beta*C with the plain triple loop over k), restated in
"How to get a matmul kernel into the top percentile (worklog)", section
"Starting Point". Sums are taken in binary64 in ascending k; every binary32
product is exact in binary64, so the oracle's own error is the binary64
summation error only, at most (K-1) * 2^-53 * sum_k |a_ik b_kj| per element.

Storage is row-major with explicit leading dimensions; ``trans`` flags are
``"N"``/``"T"`` (or 0/1). When beta == 0 the input C is not read; when
alpha == 0, A and B are not read (BLAS convention).

Parity pins for every function here live in ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import compare  # noqa: F401  (re-exported)

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_i64 = ctypes.c_int64
_dp = ctypes.POINTER(ctypes.c_double)
_fp = ctypes.POINTER(ctypes.c_float)
_ip = ctypes.POINTER(ctypes.c_int64)


def bind(path):
    """ctypes handle of an oracle shared library at ``path``."""
    lib = ctypes.CDLL(path)
    common = [ctypes.c_int, ctypes.c_int, _i64, _i64, _i64, ctypes.c_double,
              _fp, _i64, _fp, _i64, ctypes.c_double, _fp, _i64]
    lib.oracle_gemm_rows.argtypes = common + [_ip, _i64, _dp, _dp]
    lib.oracle_gemm_rows.restype = ctypes.c_int
    lib.oracle_gemm_elems.argtypes = common + [_ip, _ip, _i64, _dp, _dp]
    lib.oracle_gemm_elems.restype = ctypes.c_int
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from .build import build
        build()
    _lib = bind(_LIB_PATH)
    return _lib


def _flag(t) -> int:
    if t in (0, 1):
        return int(t)
    t = str(t).upper()
    if t not in ("N", "T"):
        raise ValueError(f"trans flag must be N or T, got {t!r}")
    return 1 if t == "T" else 0


def _as_f32(x):
    if x is None:
        return None
    x = np.ascontiguousarray(x, dtype=np.float32)
    return x


def _ptr(x, ty):
    if x is None:
        return ctypes.cast(None, ty)
    return x.ctypes.data_as(ty)


def _check_storage(name, arr, rows, cols, ld):
    """arr is a flat or 2-D float32 buffer holding a rows x cols row-major
    matrix with leading dimension ld; check that it is large enough."""
    if rows == 0 or cols == 0:
        return
    need = (rows - 1) * ld + cols
    if arr is None or arr.size < need:
        raise ValueError(f"{name}: buffer of {0 if arr is None else arr.size} "
                         f"elements cannot hold {rows}x{cols} with ld={ld}")


def _prep(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc):
    ta, tb = _flag(transA), _flag(transB)
    A, B = _as_f32(A), _as_f32(B)
    C = _as_f32(C) if beta != 0 else None
    if alpha == 0:
        return ta, tb, A, B, C
    if K > 0 and M > 0:
        _check_storage("A", A, K if ta else M, M if ta else K, lda)
    if K > 0 and N > 0:
        _check_storage("B", B, N if tb else K, K if tb else N, ldb)
    if beta != 0:
        _check_storage("C", C, M, N, ldc)
    return ta, tb, A, B, C


def gemm_rows(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C=None,
              ldc=None, rows=None, lib=None):
    """Reference rows of C_ref and S = sum_k |a_ik b_kj|, both binary64.

    ``rows`` is None (all M rows) or a sequence of row indices. Returns two
    arrays of shape (len(rows), N).
    """
    ldc = N if ldc is None else ldc
    ta, tb, A, B, C = _prep(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc)
    if rows is None:
        r = None
        nr = M
    else:
        r = np.ascontiguousarray(rows, dtype=np.int64)
        nr = r.size
    cref = np.empty((nr, N), dtype=np.float64)
    sabs = np.empty((nr, N), dtype=np.float64)
    st = (lib or _load()).oracle_gemm_rows(
        ta, tb, M, N, K, float(alpha), _ptr(A, _fp), lda, _ptr(B, _fp), ldb,
        float(beta), _ptr(C, _fp), ldc, _ptr(r, _ip), nr,
        _ptr(cref, _dp), _ptr(sabs, _dp))
    if st != 0:
        raise RuntimeError(f"oracle_gemm_rows failed with status {st}")
    return cref, sabs


def gemm(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C=None, ldc=None):
    """Whole C_ref (M x N, binary64) and S (M x N)."""
    return gemm_rows(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc)


def gemm_elems(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
               ii, jj, lib=None):
    """Reference values at the element list (ii[t], jj[t])."""
    ta, tb, A, B, C = _prep(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc)
    ii = np.ascontiguousarray(ii, dtype=np.int64)
    jj = np.ascontiguousarray(jj, dtype=np.int64)
    if ii.shape != jj.shape:
        raise ValueError("ii and jj must have the same shape")
    cref = np.empty(ii.size, dtype=np.float64)
    sabs = np.empty(ii.size, dtype=np.float64)
    st = (lib or _load()).oracle_gemm_elems(
        ta, tb, M, N, K, float(alpha), _ptr(A, _fp), lda, _ptr(B, _fp), ldb,
        float(beta), _ptr(C, _fp), ldc, _ptr(ii, _ip), _ptr(jj, _ip), ii.size,
        _ptr(cref, _dp), _ptr(sabs, _dp))
    if st != 0:
        raise RuntimeError(f"oracle_gemm_elems failed with status {st}")
    return cref, sabs


def num_threads() -> int:
    return int(_load().oracle_num_threads())

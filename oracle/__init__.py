"""CPU oracle for C = A·B in fp32 (row-major, alpha = 1, beta = 0), and for the
general form C = alpha·op(A)·op(B) + beta·C.

TEST INFRASTRUCTURE: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The GPU
library never loads it, and it loads nothing of the GPU library.

The arithmetic lives in ``sgemm_oracle.c``: the definition of the product
(page "CUDA算子优化(4)：矩阵乘法", section "矩阵乘法的数学定义"; page
"CUDA内存优化入门：从Naive到Tiled矩阵乘法—Week2学习总结", §三 and §四),
summed in double in k order.  This module only marshals numpy arrays and
applies the acceptance rule.

Acceptance rule, per element:
    |C_gpu - C| <= RTOL * S + ATOL,   S = sum_k |A[i][k]| * |B[k][j]|
with RTOL = 5e-4, the tolerance that the page "CUDA算子优化(4)：矩阵乘法"
passes to its result check, read as relative to S (that page's check routine
is not shown), and ATOL = 1e-6 for results that cancel to ~0.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

RTOL = 5e-4
ATOL = 1e-6

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sgemm_oracle.c")
_LIB = os.path.join(_HERE, "liboracle_sgemm.so")

_lib = None


def compile_flags() -> list[str]:
    return ["-O2", "-ffp-contract=off", "-fPIC", "-shared", "-pthread"]


def build(force: bool = True, src: str = _SRC, out: str = _LIB) -> str:
    """Compile the oracle with gcc (plain C, no fast-math)."""
    if force or not os.path.exists(out):
        tmp = out + ".tmp"
        subprocess.check_call(["gcc", *compile_flags(), "-o", tmp, src, "-lm"])
        os.replace(tmp, out)
    return out


def load(path: str | None = None):
    """Load the oracle library (building it first if it is absent)."""
    global _lib
    if path is None and _lib is not None:
        return _lib
    if path is None and not os.path.exists(_LIB):
        build(force=False)
    lib = ctypes.CDLL(path or _LIB)
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    lib.oracle_sgemm_f64.restype = ctypes.c_int
    lib.oracle_sgemm_f64.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, i64, vp, i64,
                                     ctypes.c_int]
    lib.oracle_sgemm_f64_elems.restype = ctypes.c_int
    lib.oracle_sgemm_f64_elems.argtypes = [i64, i64, i64, vp, i64, vp, i64, i64, vp, vp,
                                           vp, vp, ctypes.c_int]
    if hasattr(lib, "oracle_sgemm_ex_f64"):
        d, ci = ctypes.c_double, ctypes.c_int
        lib.oracle_sgemm_ex_f64.restype = ci
        lib.oracle_sgemm_ex_f64.argtypes = [ci, ci, i64, i64, i64, d, vp, i64, vp, i64, d, vp,
                                            i64, i64, vp, vp, vp, i64, vp, i64, ci]
    if path is None:
        _lib = lib
    return lib


def _threads(threads):
    if threads is not None:
        return int(threads)
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _operand(x: np.ndarray):
    """(pointer, rows, cols, ld) of a float32 2-D array with unit column stride."""
    if x.dtype != np.float32 or x.ndim != 2:
        raise TypeError("oracle operands are 2-D float32 arrays")
    rows, cols = x.shape
    if x.size == 0:
        return x.ctypes.data, rows, cols, max(cols, 1)
    if cols > 1 and x.strides[1] != 4:
        raise ValueError("oracle operands need unit column stride")
    ld = x.strides[0] // 4 if rows > 1 else cols
    if ld < cols:
        raise ValueError("oracle operands need row stride >= row length")
    return x.ctypes.data, rows, cols, ld


def sgemm(A: np.ndarray, B: np.ndarray, threads: int | None = None, lib=None):
    """Return (C, S) in float64 for C = A·B; A is M×K, B is K×N (views allowed)."""
    pa, M, K, lda = _operand(A)
    pb, K2, N, ldb = _operand(B)
    if K != K2:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    C = np.empty((M, N), dtype=np.float64)
    S = np.empty((M, N), dtype=np.float64)
    rc = (lib or load()).oracle_sgemm_f64(M, N, K, pa, lda, pb, ldb, C.ctypes.data,
                                          max(N, 1), S.ctypes.data, max(N, 1),
                                          _threads(threads))
    if rc != 0:
        raise ValueError("oracle_sgemm_f64 rejected its arguments")
    return C, S


def sgemm_elems(A: np.ndarray, B: np.ndarray, rows, cols, threads: int | None = None,
                lib=None):
    """Return (C, S) float64 vectors for the listed output elements (rows[e], cols[e])."""
    pa, M, K, lda = _operand(A)
    pb, K2, N, ldb = _operand(B)
    if K != K2:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    r = np.ascontiguousarray(rows, dtype=np.int64)
    c = np.ascontiguousarray(cols, dtype=np.int64)
    if r.shape != c.shape or r.ndim != 1:
        raise ValueError("rows and cols must be 1-D and of equal length")
    C = np.empty(r.shape[0], dtype=np.float64)
    S = np.empty(r.shape[0], dtype=np.float64)
    rc = (lib or load()).oracle_sgemm_f64_elems(M, N, K, pa, lda, pb, ldb, r.shape[0],
                                                r.ctypes.data, c.ctypes.data,
                                                C.ctypes.data, S.ctypes.data,
                                                _threads(threads))
    if rc != 0:
        raise ValueError("oracle_sgemm_f64_elems rejected its arguments")
    return C, S


def sgemm_ex(A: np.ndarray, B: np.ndarray, transa: bool = False, transb: bool = False,
             alpha: float = 1.0, beta: float = 0.0, C: np.ndarray | None = None,
             rows=None, cols=None, threads: int | None = None, lib=None):
    """Return (C_out, S) in float64 for C_out = alpha*op(A)*op(B) + beta*C.

    A and B are the stored arrays: op(A) is A (M x K) or, with transa, the
    transpose of the K x M array A; op(B) is B (K x N) or, with transb, the
    transpose of the N x K array B.  C (M x N float32) is read only when
    beta != 0.  alpha and beta are rounded to float32 first, as the GPU
    boundary takes them.  With rows/cols, only the listed elements are
    computed and returned as vectors.
    """
    pa, ra, ca, lda = _operand(A)
    pb, rb, cb, ldb = _operand(B)
    M, K = (ca, ra) if transa else (ra, ca)
    K2, N = (cb, rb) if transb else (rb, cb)
    if K != K2:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    alpha = float(np.float32(alpha))
    beta = float(np.float32(beta))
    pc, ldcin = 0, max(N, 1)
    if beta != 0.0 and C is None:
        raise ValueError("beta != 0 needs C")
    if C is not None:
        pc, rc_, cc_, ldcin = _operand(C)
        if (rc_, cc_) != (M, N):
            raise ValueError("C has the wrong shape")
    fn = (lib or load()).oracle_sgemm_ex_f64
    if rows is None:
        out = np.empty((M, N), dtype=np.float64)
        S = np.empty((M, N), dtype=np.float64)
        rc = fn(int(transa), int(transb), M, N, K, alpha, pa, lda, pb, ldb, beta, pc, ldcin,
                0, None, None, out.ctypes.data, max(N, 1), S.ctypes.data, max(N, 1),
                _threads(threads))
    else:
        r = np.ascontiguousarray(rows, dtype=np.int64)
        c = np.ascontiguousarray(cols, dtype=np.int64)
        if r.shape != c.shape or r.ndim != 1:
            raise ValueError("rows and cols must be 1-D and of equal length")
        out = np.empty(r.shape[0], dtype=np.float64)
        S = np.empty(r.shape[0], dtype=np.float64)
        rc = fn(int(transa), int(transb), M, N, K, alpha, pa, lda, pb, ldb, beta, pc, ldcin,
                r.shape[0], r.ctypes.data, c.ctypes.data, out.ctypes.data, 0, S.ctypes.data, 0,
                _threads(threads))
    if rc != 0:
        raise ValueError("oracle_sgemm_ex_f64 rejected its arguments")
    return out, S


def excess(C_gpu: np.ndarray, C: np.ndarray, S: np.ndarray) -> np.ndarray:
    """|C_gpu - C| / (RTOL*S + ATOL), evaluated in float64; <= 1 means accepted.

    Non-finite GPU values count as infinitely wrong unless the oracle's value
    is the same non-finite value.
    """
    g = np.asarray(C_gpu, dtype=np.float64)
    with np.errstate(invalid="ignore"):
        diff = np.abs(g - C)
        out = diff / (RTOL * S + ATOL)
    same_nonfinite = ~np.isfinite(g) & (g == C)
    out = np.where(same_nonfinite, 0.0, out)
    out = np.where(np.isnan(out), np.inf, out)
    return out


def accept(C_gpu: np.ndarray, C: np.ndarray, S: np.ndarray) -> bool:
    """True iff every element satisfies the acceptance rule."""
    return bool(np.all(excess(C_gpu, C, S) <= 1.0))

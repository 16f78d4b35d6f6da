"""Cache-blocked, multi-threaded fp32 matrix product on the host CPU.

A host baseline for timing next to the oracle: the pages' serial CPU loop
(page "CUDA内存优化入门：从Naive到Tiled矩阵乘法—Week2学习总结", §四) rearranged for a
multi-core CPU (row ranges per thread, packed k panels, a register-blocked
micro-kernel).  It shares no code with the oracle or the GPU library, and
neither of them uses it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hostsgemm.c")
_LIB = os.path.join(_HERE, "libhostsgemm.so")
_lib = None


def compile_flags() -> list[str]:
    # x86-64-v3 (AVX2 + FMA): available on every current server CPU
    return ["-O3", "-march=x86-64-v3", "-fPIC", "-shared", "-pthread"]


def build(force: bool = True) -> str:
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", *compile_flags(), "-o", tmp, _SRC])
        os.replace(tmp, _LIB)
    return _LIB


def load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        i64, vp = ctypes.c_int64, ctypes.c_void_p
        lib.host_sgemm.restype = ctypes.c_int
        lib.host_sgemm.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, i64, ctypes.c_int]
        _lib = lib
    return _lib


def threads_available() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def sgemm(A: np.ndarray, B: np.ndarray, threads: int | None = None) -> np.ndarray:
    """C = A·B in float32 for 2-D float32 arrays with unit column stride."""
    for x in (A, B):
        if x.dtype != np.float32 or x.ndim != 2:
            raise TypeError("operands are 2-D float32 arrays")
        if x.size > 0 and x.shape[1] > 1 and x.strides[1] != 4:
            raise ValueError("operands need unit column stride")
    M, K = A.shape
    K2, N = B.shape
    if K != K2:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    C = np.empty((M, N), dtype=np.float32)
    if A.size == 0 or B.size == 0:
        C[...] = 0.0
        return C
    lda = A.strides[0] // 4 if M > 1 else max(K, 1)
    ldb = B.strides[0] // 4 if K > 1 else max(N, 1)
    rc = load().host_sgemm(M, N, K, A.ctypes.data, max(lda, K, 1), B.ctypes.data,
                           max(ldb, N, 1), C.ctypes.data, max(N, 1),
                           threads if threads is not None else threads_available())
    if rc != 0:
        raise RuntimeError("host_sgemm failed")
    return C

"""Seeded synthetic inputs shared by the GPU path's tests/bench and the CPU oracle.

This package only draws numbers (see ``synthgen.c`` for the generator's
definition); it holds none of the matrix product's arithmetic, so both sides
of a parity check may use it without sharing any of the method's code.

Input recipes follow the workloads of the pages: square products with
N(0,1) entries (page "CUDA算子优化(4)：矩阵乘法", its two test programs draw
A and B from a normal distribution), uniform entries (page
"CUDA内存优化入门：从Naive到Tiled矩阵乘法—Week2学习总结", §八 initialises with
uniform random values), and all-ones matrices (page "GPU programming with C++
and CUDA", chapter 7, examples 1 and 2).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synthgen.c")
_LIB = os.path.join(_HERE, "libsynthgen.so")

DISTS = {"normal": 0, "uniform_pm1": 1, "smallint": 2, "uniform01": 3}

_lib = None


def build(force: bool = True) -> str:
    """Compile libsynthgen.so with gcc (host code only)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-fPIC", "-shared", "-pthread", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        lib.synth_fill_f32.restype = ctypes.c_int
        lib.synth_fill_f32.argtypes = [
            ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int, ctypes.c_int]
        lib.synth_word.restype = ctypes.c_uint64
        lib.synth_word.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64]
        lib.synth_key.restype = ctypes.c_uint64
        lib.synth_key.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
        _lib = lib
    return _lib


def host_threads() -> int:
    """Threads this process may run on (affinity mask, not the machine size)."""
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def word(seed: int, stream: int, counter: int) -> int:
    """Raw 64-bit word `counter` of stream (seed, stream)."""
    return int(_load().synth_word(seed, stream, counter))


def matrix(rows: int, cols: int, *, seed: int, stream: int, dist: str = "normal",
           ld: int | None = None, pad_value: float = float("nan"),
           threads: int | None = None) -> np.ndarray:
    """Return a (rows, ld) float32 array whose [:, :cols] part is the seeded matrix.

    Columns cols..ld-1 (row padding) hold ``pad_value`` so that a kernel which
    reads past a row's logical end shows up as a non-finite result.
    """
    ld = cols if ld is None else int(ld)
    if ld < cols:
        raise ValueError("ld must be >= cols")
    out = np.empty((rows, max(ld, 1)), dtype=np.float32)
    if ld > cols:
        out[:, cols:] = pad_value
    rc = _load().synth_fill_f32(
        out.ctypes.data, rows, cols, max(ld, 1), seed, stream, DISTS[dist],
        threads if threads is not None else host_threads())
    if rc != 0:
        raise ValueError("synth_fill_f32 rejected its arguments")
    return out


def ones(rows: int, cols: int, ld: int | None = None) -> np.ndarray:
    ld = cols if ld is None else ld
    out = np.full((rows, max(ld, 1)), np.nan, dtype=np.float32)
    out[:, :cols] = 1.0
    return out


def identity(n: int) -> np.ndarray:
    return np.eye(n, dtype=np.float32)

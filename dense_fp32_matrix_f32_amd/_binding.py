"""ctypes binding of include/sgemm_f32.h: the same entry points, same arguments.

This layer only marshals arguments.  Every step of the product runs in the HIP
kernels of libsgemm_f32.so; there is no fallback of any kind, and a missing
library is an error.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsgemm_f32.so")

ALGO_AUTO = 0
ALGO_NAIVE = 1
ALGO_LDS_TILED = 2
ALGO_VALU_REGBLOCK = 3
ALGO_MFMA = 4
ALGO_SKINNY = 5
ALGO_SKINNY_N = 6
ALGO_BF16X6 = 7
ALGO_COUNT = 8
ALGOS = {"auto": ALGO_AUTO, "naive": ALGO_NAIVE, "lds_tiled": ALGO_LDS_TILED,
         "valu_regblock": ALGO_VALU_REGBLOCK, "mfma": ALGO_MFMA, "skinny": ALGO_SKINNY,
         "skinny_n": ALGO_SKINNY_N, "bf16x6": ALGO_BF16X6}

HIP_SUCCESS = 0
HIP_ERROR_INVALID_VALUE = 1

OP_N = 0
OP_T = 1

EXPORTED = ("sgemm_f32", "sgemm_f32_algo", "sgemm_f32_select", "sgemm_f32_algo_name",
            "sgemm_f32_ex", "sgemm_f32_ex_algo", "sgemm_f32_colmajor",
            "sgemm_f32_mfma_tiles", "sgemm_f32_mfma_tile_name", "sgemm_f32_mfma_select",
            "sgemm_f32_mfma_tile", "sgemm_f32_ex_mfma_tile", "sgemm_f32_auto_plan",
            "sgemm_f32_workspace_size", "sgemm_f32_ex_ws", "sgemm_f32_ex_noalloc")

SCRATCH_BYTES = 32 << 20   # SGEMM_F32_SCRATCH_BYTES

_lib = None


class SgemmError(RuntimeError):
    def __init__(self, status: int, what: str = "sgemm_f32"):
        super().__init__(f"{what} returned hipError_t {status}")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded C-ABI library; raises if it has not been built."""
    global _lib
    if _lib is None:
        # torch ships its own HIP runtime under the same soname as ROCm's.  Load it
        # first so that this library binds to it: one runtime per process, which is
        # what makes torch's device pointers and stream handles valid here.
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                "(hipcc, gfx950); there is no other implementation")
        l = ctypes.CDLL(LIB_PATH)
        i, vp = ctypes.c_int, ctypes.c_void_p
        args = [i, i, i, vp, i, vp, i, vp, i, vp]
        l.sgemm_f32.argtypes = args
        l.sgemm_f32.restype = i
        l.sgemm_f32_algo.argtypes = args + [i]
        l.sgemm_f32_algo.restype = i
        l.sgemm_f32_select.argtypes = [i, i, i, vp, i, vp, i, vp, i]
        l.sgemm_f32_select.restype = i
        l.sgemm_f32_algo_name.argtypes = [i]
        l.sgemm_f32_algo_name.restype = ctypes.c_char_p
        l.sgemm_f32_mfma_tiles.argtypes = []
        l.sgemm_f32_mfma_tiles.restype = i
        l.sgemm_f32_mfma_tile_name.argtypes = [i]
        l.sgemm_f32_mfma_tile_name.restype = ctypes.c_char_p
        l.sgemm_f32_mfma_select.argtypes = [i, i, i, i]
        l.sgemm_f32_mfma_select.restype = i
        l.sgemm_f32_mfma_tile.argtypes = args + [i]
        l.sgemm_f32_mfma_tile.restype = i
        f = ctypes.c_float
        ex_args = [i, i, i, i, i, f, vp, i, vp, i, f, vp, i, vp]
        for name in ("sgemm_f32_ex", "sgemm_f32_colmajor"):
            getattr(l, name).argtypes = ex_args
            getattr(l, name).restype = i
        l.sgemm_f32_ex_algo.argtypes = ex_args + [i]
        l.sgemm_f32_ex_algo.restype = i
        l.sgemm_f32_ex_mfma_tile.argtypes = ex_args + [i]
        l.sgemm_f32_ex_mfma_tile.restype = i
        l.sgemm_f32_workspace_size.argtypes = [i, i, i, i, i]
        l.sgemm_f32_workspace_size.restype = ctypes.c_size_t
        l.sgemm_f32_ex_ws.argtypes = [i, i, i, i, i, f, vp, i, vp, i, f, vp, i, vp, ctypes.c_size_t,
                                      vp]
        l.sgemm_f32_ex_ws.restype = i
        l.sgemm_f32_ex_noalloc.argtypes = ex_args
        l.sgemm_f32_ex_noalloc.restype = i
        ip = ctypes.POINTER(i)
        l.sgemm_f32_auto_plan.argtypes = [i, i, i, i, i, i, ip, ip]
        l.sgemm_f32_auto_plan.restype = i
        _lib = l
    return _lib


def sgemm_f32(M, N, K, A, lda, B, ldb, C, ldc, stream=0) -> int:
    """C = A·B; pointers are device addresses (int); returns the hipError_t."""
    return lib().sgemm_f32(M, N, K, A, lda, B, ldb, C, ldc, stream)


def sgemm_f32_algo(M, N, K, A, lda, B, ldb, C, ldc, stream=0, algo=ALGO_AUTO) -> int:
    """As sgemm_f32 with a forced algorithm id; returns the hipError_t."""
    return lib().sgemm_f32_algo(M, N, K, A, lda, B, ldb, C, ldc, stream, algo)


def sgemm_f32_select(M, N, K, A, lda, B, ldb, C, ldc) -> int:
    """Algorithm id AUTO would use (host-only), or -1 for invalid arguments."""
    return lib().sgemm_f32_select(M, N, K, A, lda, B, ldb, C, ldc)


def sgemm_f32_algo_name(algo: int) -> str:
    return lib().sgemm_f32_algo_name(algo).decode()


def sgemm_f32_mfma_tiles() -> int:
    """Number of tile configurations of the matrix-core rung."""
    return lib().sgemm_f32_mfma_tiles()


def sgemm_f32_mfma_tile_name(tile: int):
    """Description of configuration `tile`, or None for an unknown id."""
    r = lib().sgemm_f32_mfma_tile_name(tile)
    return None if r is None else r.decode()


def sgemm_f32_mfma_select(M, N, K, compute_units=256) -> int:
    """Configuration id the matrix-core rung uses for this shape (host-only)."""
    return lib().sgemm_f32_mfma_select(M, N, K, compute_units)


def sgemm_f32_auto_plan(transa, transb, M, N, K, compute_units=256):
    """(algorithm id, m_main, n_main) of the automatic choice (host-only); the id is
    -1 for invalid arguments.  Columns [n_main, N) and then rows [m_main, M) of
    columns [0, n_main) go to a second kernel sized for that strip."""
    m, n = ctypes.c_int(-1), ctypes.c_int(-1)
    algo = lib().sgemm_f32_auto_plan(transa, transb, M, N, K, compute_units,
                                     ctypes.byref(m), ctypes.byref(n))
    return algo, m.value, n.value


def sgemm_f32_workspace_size(transa, transb, M, N, K) -> int:
    """Bytes of workspace sgemm_f32_ex_ws would use (0: no split); no GPU work."""
    return lib().sgemm_f32_workspace_size(transa, transb, M, N, K)


def sgemm_f32_ex_ws(transa, transb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, workspace,
                    workspace_bytes, stream=0) -> int:
    """sgemm_f32_ex with a device workspace (split-k when it pays); returns the hipError_t."""
    return lib().sgemm_f32_ex_ws(transa, transb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                                 workspace, workspace_bytes, stream)


def sgemm_f32_ex_noalloc(transa, transb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                         stream=0) -> int:
    """sgemm_f32_ex_ws with the library's own device scratch array as the workspace
    (allocates nothing); returns the hipError_t."""
    return lib().sgemm_f32_ex_noalloc(transa, transb, M, N, K, alpha, A, lda, B, ldb, beta, C,
                                      ldc, stream)


def sgemm_f32_mfma_tile(M, N, K, A, lda, B, ldb, C, ldc, stream=0, tile=0) -> int:
    """C = A·B on the matrix-core rung with configuration `tile`; returns the hipError_t."""
    return lib().sgemm_f32_mfma_tile(M, N, K, A, lda, B, ldb, C, ldc, stream, tile)


def sgemm_f32_ex(transa, transb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=0) -> int:
    """C = alpha*op(A)*op(B) + beta*C (row-major); returns the hipError_t."""
    return lib().sgemm_f32_ex(transa, transb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                              stream)


def sgemm_f32_ex_algo(transa, transb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=0,
                      algo=ALGO_AUTO) -> int:
    """As sgemm_f32_ex with a forced algorithm id; returns the hipError_t."""
    return lib().sgemm_f32_ex_algo(transa, transb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                                   stream, algo)


def sgemm_f32_colmajor(transa, transb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                       stream=0) -> int:
    """The general form with column-major arrays (reference-BLAS argument order)."""
    return lib().sgemm_f32_colmajor(transa, transb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                                    stream)


def sgemm_f32_ex_mfma_tile(transa, transb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                           stream=0, tile=0) -> int:
    """The general form on the matrix-core rung with configuration `tile`."""
    return lib().sgemm_f32_ex_mfma_tile(transa, transb, M, N, K, alpha, A, lda, B, ldb, beta, C,
                                        ldc, stream, tile)

"""Single-precision matrix product C = A·B on MI355X (gfx950), behind a C ABI.

The library (``libsgemm_f32.so``, built from ``csrc/`` by ``build.py``) exports
the entry points of ``include/sgemm_f32.h``; ``_binding`` mirrors them one to
one.  ``matmul`` is a convenience for torch tensors: torch provides the device
memory and the stream, the library does all of the arithmetic.
"""
from __future__ import annotations

from ._binding import (ALGO_AUTO, ALGO_COUNT, ALGO_LDS_TILED, ALGO_MFMA, ALGO_NAIVE,
                       ALGO_SKINNY, ALGO_SKINNY_N, ALGO_VALU_REGBLOCK, ALGOS, EXPORTED, LIB_PATH,
                       SgemmError, lib, sgemm_f32, sgemm_f32_algo, sgemm_f32_algo_name,
                       sgemm_f32_mfma_select, sgemm_f32_mfma_tile, sgemm_f32_mfma_tile_name,
                       sgemm_f32_mfma_tiles, sgemm_f32_select)

__all__ = ["matmul", "sgemm_f32", "sgemm_f32_algo", "sgemm_f32_select", "sgemm_f32_algo_name",
           "sgemm_f32_mfma_tiles", "sgemm_f32_mfma_tile_name", "sgemm_f32_mfma_select",
           "sgemm_f32_mfma_tile", "SgemmError", "ALGOS", "LIB_PATH", "EXPORTED", "lib"]


def _operand(t, name):
    import torch
    if not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or t.dim() != 2:
        raise TypeError(f"{name} must be a 2-D float32 torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live on the GPU")
    if t.numel() > 0 and t.size(1) > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} needs unit column stride (row-major)")
    ld = t.stride(0) if t.size(0) > 1 else t.size(1)
    return t.data_ptr(), max(ld, t.size(1), 1)


def matmul(A, B, out=None, algo="auto", stream=None):
    """Return C = A @ B for 2-D float32 CUDA tensors (row-major; views with a row
    stride are passed as leading dimensions).  Enqueued on ``stream`` (default:
    torch's current stream) without synchronising."""
    import torch
    pa, lda = _operand(A, "A")
    pb, ldb = _operand(B, "B")
    M, K = A.shape
    K2, N = B.shape
    if K != K2:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=A.device)
    elif tuple(out.shape) != (M, N):
        raise ValueError("out has the wrong shape")
    pc, ldc = _operand(out, "out")
    s = stream if stream is not None else torch.cuda.current_stream(A.device)
    algo_id = ALGOS[algo] if isinstance(algo, str) else int(algo)
    with torch.cuda.device(A.device):
        st = sgemm_f32_algo(M, N, K, pa, lda, pb, ldb, pc, ldc, s.cuda_stream, algo_id)
    if st != 0:
        raise SgemmError(st)
    return out

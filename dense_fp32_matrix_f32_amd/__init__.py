"""Single-precision matrix product C = A·B on MI355X (gfx950), behind a C ABI.

The library (``libsgemm_f32.so``, built from ``csrc/`` by ``build.py``) exports
the entry points of ``include/sgemm_f32.h``; ``_binding`` mirrors them one to
one.  ``matmul`` is a convenience for torch tensors: torch provides the device
memory and the stream, the library does all of the arithmetic.
"""
from __future__ import annotations

from ._binding import (ALGO_AUTO, ALGO_BF16X6, ALGO_COUNT, ALGO_LDS_TILED, ALGO_MFMA, ALGO_NAIVE,
                       ALGO_SKINNY, ALGO_SKINNY_N, ALGO_VALU_REGBLOCK, ALGOS, EXPORTED, LIB_PATH,
                       OP_N, OP_T, SgemmError, lib, sgemm_f32, sgemm_f32_algo, sgemm_f32_algo_name,
                       sgemm_f32_colmajor, sgemm_f32_ex, sgemm_f32_ex_algo,
                       sgemm_f32_ex_mfma_tile, sgemm_f32_mfma_select, sgemm_f32_mfma_tile,
                       sgemm_f32_mfma_tile_name, sgemm_f32_mfma_tiles, sgemm_f32_select,
                       sgemm_f32_auto_plan, sgemm_f32_ex_ws, sgemm_f32_workspace_size,
                       sgemm_f32_ex_noalloc, SCRATCH_BYTES)

__all__ = ["matmul", "sgemm_f32", "sgemm_f32_algo", "sgemm_f32_select", "sgemm_f32_algo_name",
           "sgemm_f32_ex", "sgemm_f32_ex_algo", "sgemm_f32_colmajor", "sgemm_f32_mfma_tiles",
           "sgemm_f32_mfma_tile_name", "sgemm_f32_mfma_select", "sgemm_f32_mfma_tile",
           "sgemm_f32_ex_mfma_tile", "sgemm_f32_auto_plan", "sgemm_f32_workspace_size", "sgemm_f32_ex_ws",
           "sgemm_f32_ex_noalloc", "SCRATCH_BYTES", "SgemmError", "ALGOS", "LIB_PATH", "EXPORTED", "lib",
           "OP_N", "OP_T"]


def _layout(rows, cols, s0, s1, name):
    """(leading dimension, transposed) of a rows x cols view with element strides
    (s0, s1): row-major when its column stride is 1, the transpose of a row-major
    array when its row stride is 1.  A stride shorter than the row it steps over
    (a broadcast or overlapping view, e.g. ``expand``) is rejected: the library
    would read or write past the view's memory with the leading dimension it
    implies."""
    if rows == 0 or cols == 0:
        return max(cols, 1), False
    if cols == 1 or s1 == 1:
        if rows > 1 and s0 < cols:
            raise ValueError(f"{name}: row stride {s0} is shorter than a row ({cols}); "
                             "broadcast or overlapping views are not supported")
        return (s0 if rows > 1 else cols), False
    if rows == 1 or s0 == 1:
        if s1 < rows:
            raise ValueError(f"{name}: column stride {s1} is shorter than a column ({rows}); "
                             "broadcast or overlapping views are not supported")
        return s1, True
    raise ValueError(f"{name} needs a unit stride in one dimension")


def _operand(t, name):
    """(pointer, leading dimension, transposed) of a 2-D float32 CUDA tensor that is
    row-major (unit column stride) or the transpose of a row-major array (unit row
    stride, e.g. ``X.t()``)."""
    import torch
    if not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or t.dim() != 2:
        raise TypeError(f"{name} must be a 2-D float32 torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live on the GPU")
    rows, cols = t.shape
    ld, trans = _layout(rows, cols, t.stride(0), t.stride(1), name)
    return t.data_ptr(), ld, trans


def matmul(A, B, out=None, algo="auto", stream=None, alpha=1.0, beta=0.0, workspace=None):
    """Return C = alpha * A @ B + beta * out for 2-D float32 CUDA tensors.

    Row-major tensors and views with a row stride are passed as they are;
    transposed views (``X.t()``) are passed as transposed operands, without a
    copy.  ``out`` must be row-major; it is read only when beta != 0 (a new
    tensor is allocated when it is None, which needs beta == 0).  With algo
    "auto", ``workspace`` (a contiguous CUDA tensor, or "auto" to allocate the
    size sgemm_f32_workspace_size asks for through torch) lets products with few
    blocks of C split k across work-groups.  The product is enqueued on
    ``stream`` (default: torch's current stream) without synchronising; tensors
    allocated here (``out`` when None, the "auto" workspace) are marked as used on
    that stream, so torch's allocator does not hand their memory out again before
    the product has finished there."""
    import torch
    pa, lda, ta = _operand(A, "A")
    pb, ldb, tb = _operand(B, "B")
    M, K = A.shape
    K2, N = B.shape
    if K != K2:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    made = []  # tensors allocated here, to be marked as used on the launch stream
    if out is None:
        if beta != 0.0:
            raise ValueError("beta != 0 needs out")
        out = torch.empty((M, N), dtype=torch.float32, device=A.device)
        made.append(out)
    elif tuple(out.shape) != (M, N):
        raise ValueError("out has the wrong shape")
    pc, ldc, tc = _operand(out, "out")
    if tc and M > 1 and N > 1:
        raise ValueError("out must be row-major")
    s = stream if stream is not None else torch.cuda.current_stream(A.device)
    algo_id = ALGOS[algo] if isinstance(algo, str) else int(algo)
    with torch.cuda.device(A.device):
        if workspace is not None and algo_id == ALGO_AUTO:
            if isinstance(workspace, str):
                if workspace != "auto":
                    raise ValueError('workspace must be a tensor, "auto" or None')
                nbytes = sgemm_f32_workspace_size(int(ta), int(tb), M, N, K)
                workspace = torch.empty(max(nbytes // 4, 1), dtype=torch.float32, device=A.device)
                made.append(workspace)
            if not workspace.is_cuda or not workspace.is_contiguous():
                raise ValueError("workspace must be a contiguous CUDA tensor")
            st = sgemm_f32_ex_ws(int(ta), int(tb), M, N, K, float(alpha), pa, lda, pb, ldb,
                                 float(beta), pc, ldc, workspace.data_ptr(),
                                 workspace.numel() * workspace.element_size(), s.cuda_stream)
        else:
            st = sgemm_f32_ex_algo(int(ta), int(tb), M, N, K, float(alpha), pa, lda, pb, ldb,
                                   float(beta), pc, ldc, s.cuda_stream, algo_id)
    if st != 0:
        raise SgemmError(st)
    if isinstance(s, torch.cuda.Stream):
        for t in made:
            t.record_stream(s)
    return out

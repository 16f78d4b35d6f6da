"""Every tile configuration of the matrix-core rung against the oracle.

The automatic choice reaches each configuration only on some shapes, so each one
is forced here through sgemm_f32_mfma_tile() on shapes built from its own block
sizes: whole blocks only, ragged right and bottom edges with a partial last k
window, fewer than four columns, row strides beyond the row length with 4-byte
alignment, and a product long enough in k for the steady-state loop of both the
interior and the right-edge work-groups.  Small-integer inputs make every
correct summation order exact, so those cases are compared bitwise.
"""
import re

import pytest

import dense_fp32_matrix_f32_amd as sg
from gpu_helpers import Device, assert_guards, check_full, inputs, log

pytestmark = pytest.mark.gpu

TILES = list(range(sg.sgemm_f32_mfma_tiles()))


def _blocks(tile):
    bm, bn, bk = map(int, re.match(r"(\d+)x(\d+)x(\d+)", sg.sgemm_f32_mfma_tile_name(tile)).groups())
    return bm, bn, bk


def _run(tile, A, B, M, N, K, **kw):
    log(f"[gpu] mfma tile {sg.sgemm_f32_mfma_tile_name(tile)} M={M} N={N} K={K} "
        f"lda={A.shape[1]} ldb={B.shape[1]} {kw}")
    d = Device(A, B, M, N, K, **kw)
    d.run_tile(tile)
    C, guards = d.result()
    assert_guards(guards)
    return C


def _shapes(tile):
    bm, bn, bk = _blocks(tile)
    return {
        "whole": (2 * bm, 2 * bn, 12 * bk),
        "ragged": (2 * bm + 37, 2 * bn + 19, 9 * bk + 3),
        "few_columns": (bm + 1, 3, 6 * bk + 1),
        "one_block": (bm - 5, bn - 7, bk - 1),
    }


@pytest.mark.parametrize("case", ["whole", "ragged", "few_columns", "one_block"])
@pytest.mark.parametrize("tile", TILES, ids=sg.sgemm_f32_mfma_tile_name)
def test_tile_exact_integers(tile, case):
    M, N, K = _shapes(tile)[case]
    A, B = inputs(M, N, K, "smallint", seed=300 + tile)
    C = _run(tile, A, B, M, N, K)
    check_full(A, B, M, N, K, C, f"tile {tile} {case}", exact=True)


@pytest.mark.parametrize("tile", TILES, ids=sg.sgemm_f32_mfma_tile_name)
def test_tile_normal_padded_misaligned(tile):
    bm, bn, bk = _blocks(tile)
    M, N, K = bm + 3, 2 * bn + 5, 7 * bk + 2
    A, B = inputs(M, N, K, "normal", seed=400 + tile, lda=K + 5, ldb=N + 3)
    C = _run(tile, A, B, M, N, K, ldc=N + 7, offset_elems=1)
    check_full(A, B, M, N, K, C, f"tile {tile} padded")


@pytest.mark.parametrize("tile", TILES, ids=sg.sgemm_f32_mfma_tile_name)
def test_tile_k_zero_and_empty(tile):
    A, B = inputs(5, 6, 1, "normal", seed=1)
    C = _run(tile, A, B, 5, 6, 0)
    assert (C == 0).all()


# Row strides so long that some lane of a block lies 2^31 bytes or more from the
# block's first row or column: the kernels (matrix-core and split-precision
# rungs) then address with 64-bit per-lane pointers instead of 32-bit offsets
# from a uniform base.  (layout, M, N, K, lda,
# ldb) with the stored arrays' row counts: A is M x lda (K x lda transposed), B is
# K x ldb (N x ldb transposed).  Only the logical columns are copied to the GPU.
WIDE = [
    ((0, 0), 64, 48, 40, 2_200_000, 48),        # A k-contiguous, 255 rows apart
    ((0, 0), 64, 48, 16, 40, 36_000_000),       # B n-contiguous, 15 rows apart
    ((1, 1), 64, 48, 16, 36_000_000, 2_200_000),  # both transposed
    ((0, 0), 64, 48, 40, 18_000_000, 48),       # A k-contiguous, 31 rows apart (32-row blocks)
]


@pytest.mark.parametrize("case", WIDE, ids=lambda c: f"{'T' if c[0][0] else 'N'}"
                         f"{'T' if c[0][1] else 'N'}-lda{c[4]}-ldb{c[5]}")
def test_wide_row_strides(case):
    import numpy as np
    import torch

    import oracle
    import synthgen
    (ta, tb), M, N, K, lda, ldb = case
    X = synthgen.matrix(M, K, seed=61, stream=0, dist="smallint")   # op(A)
    Y = synthgen.matrix(K, N, seed=61, stream=1, dist="smallint")   # op(B)
    As = np.ascontiguousarray(X.T if ta else X)
    Bs = np.ascontiguousarray(Y.T if tb else Y)
    exact, _ = oracle.sgemm(X, Y)
    dev = {}
    for name, S, ld in (("A", As, lda), ("B", Bs, ldb)):
        buf = torch.zeros(S.shape[0] * ld, dtype=torch.float32, device="cuda")
        buf.view(S.shape[0], ld)[:, :S.shape[1]] = torch.from_numpy(S).cuda()
        dev[name] = buf
    stream = torch.cuda.current_stream()
    try:
        # every tile forced, the automatic tile, and (untransposed only) the split rung
        runs = list(range(sg.sgemm_f32_mfma_tiles())) + [None] + \
            (["bf16x6"] if (ta, tb) == (0, 0) else [])
        for tile in runs:
            C = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
            log(f"[gpu] wide strides {'T' if ta else 'N'}{'T' if tb else 'N'} tile={tile} "
                f"M={M} N={N} K={K} lda={lda} ldb={ldb}")
            args = (ta, tb, M, N, K, 1.0, dev["A"].data_ptr(), lda, dev["B"].data_ptr(), ldb, 0.0,
                    C.data_ptr(), N, stream.cuda_stream)
            if tile == "bf16x6":
                st = sg.sgemm_f32_ex_algo(*args, sg.ALGO_BF16X6)
            elif tile is not None:
                st = sg.sgemm_f32_ex_mfma_tile(*args, tile)
            else:
                st = sg.sgemm_f32_ex_algo(*args, sg.ALGO_MFMA)
            assert st == 0
            stream.synchronize()
            assert np.array_equal(C.cpu().numpy().astype(np.float64), exact), f"tile {tile}"
    finally:
        del dev
        torch.cuda.empty_cache()

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

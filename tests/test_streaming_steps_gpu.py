"""The streaming kernels' k schedules at the lengths where they change shape.

Few rows with x contiguous along k take runs of four consecutive k per slot,
with the last run of a slot cut by K (K = 1 to 7, K just past a multiple of four
or of 4*slots), on 512 or 256 work-items depending on the number of column
strips (and 64-column strips from 16384 columns on).  Few columns with y read
along k, or two dense columns of y, issue the loads of four or eight steps of 256
k at once (four from K = 769, eight from K = 2048), with the remaining steps
and the last partial piece of each lane taken one at a time.  Every case runs
on small integers with integer alpha and beta, so the result is exact and is
compared bitwise with the oracle; A's row stride is also padded to an odd
length and the operands moved off 16-byte alignment.
"""
import numpy as np
import pytest

import dense_fp32_matrix_f32_amd as sg
import synthgen
from gpu_helpers import Device, assert_guards, check_ex, log, stored

pytestmark = pytest.mark.gpu

N_, T_ = sg.OP_N, sg.OP_T
name = sg.sgemm_f32_algo_name


def _case(M, N, K, ta, tb, seed, algo, pad_a=0, offset=0):
    X = synthgen.matrix(M, K, seed=seed, stream=0, dist="smallint")
    Y = synthgen.matrix(K, N, seed=seed, stream=1, dist="smallint")
    C0 = synthgen.matrix(M, N, seed=seed, stream=2, dist="smallint")
    As = stored(X, ta, (M if ta else K) + pad_a if pad_a else None)
    Bs = stored(Y, tb)
    tag = f"{'T' if ta else 'N'}{'T' if tb else 'N'} {name(algo)} {M}x{N}x{K} pad {pad_a} off {offset}"
    log(f"[gpu] streaming steps {tag}")
    d = Device(As, Bs, M, N, K, c_init=C0, offset_elems=offset)
    d.run_ex(ta, tb, 2.0, -1.0, algo=algo)
    C, guards = d.result()
    assert_guards(guards)
    check_ex(As, Bs, M, N, K, ta, tb, 2.0, -1.0, C0, C, tag, exact=True)


# Few rows, x = op(A) contiguous along k (A as given): runs of four k.
RUN_K = [1, 2, 3, 4, 5, 7, 255, 257, 1023, 1027, 2049, 4099]


@pytest.mark.parametrize("K", RUN_K)
@pytest.mark.parametrize("M", [1, 3, 8])
def test_few_rows_runs_of_four(M, K):
    # 4096 columns: 256 strips of 16 (512 work-items); 5000: 313 strips (256)
    for N in (4096, 5000):
        _case(M, N, K, N_, N_, 40 + M + K, sg.ALGO_AUTO)
    _case(M, 1000, K, N_, N_, 50 + M + K, sg.ALGO_SKINNY, pad_a=3, offset=1)


@pytest.mark.parametrize("N", [16384, 17000])
def test_few_rows_runs_of_four_wide_strips(N):
    # 64-column strips: 256 of them (512 work-items), or 266 (256 work-items)
    for M, K in [(1, 301), (2, 1027), (5, 6)]:
        _case(M, N, K, N_, N_, 60 + M + K, sg.ALGO_AUTO)


@pytest.mark.parametrize("K", [3, 5, 1027, 4099])
def test_few_columns_both_transposed_runs_of_four(K):
    # few columns with both operands transposed: x = op(B)^T, contiguous along k
    for (M, N) in [(4096, 1), (700, 3), (1001, 8)]:
        _case(M, N, K, T_, T_, 70 + N + K, sg.ALGO_AUTO)


# Few columns, y read along k or two dense columns: batches of four or eight
# steps of 256 k.
BATCH_K = [700, 769, 1000, 1023, 1025, 2047, 2048, 2049, 2303, 4097, 6000]


@pytest.mark.parametrize("K", BATCH_K)
def test_few_columns_batches_y_along_k(K):
    # B transposed: y = op(B) with its columns contiguous along k
    for (M, N) in [(1001, 1), (513, 2), (300, 4), (257, 3)]:
        _case(M, N, K, N_, T_, 80 + N + K, sg.ALGO_AUTO)
    _case(777, 2, K, N_, T_, 85 + K, sg.ALGO_SKINNY_N, pad_a=5, offset=1)


@pytest.mark.parametrize("K", BATCH_K)
def test_few_rows_times_transposed_matrix_batches(K):
    # x * W^T: few rows with B transposed stream the stored N x K array B, with
    # y = op(A)^T read along k
    for (M, N) in [(1, 4096), (2, 1000), (4, 333)]:
        _case(M, N, K, N_, T_, 90 + M + K, sg.ALGO_AUTO)


@pytest.mark.parametrize("K", [769, 1025, 2048, 2049, 4097])
def test_few_columns_batches_two_dense_columns(K):
    # N = 2 with B dense (ldb = 2): a lane's four rows of y are eight floats
    for M in (1000, 4096):
        _case(M, 2, K, N_, N_, 95 + M + K, sg.ALGO_AUTO)

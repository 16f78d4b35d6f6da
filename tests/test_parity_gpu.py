"""Parity of the HIP kernels with the CPU oracle, called through the C ABI.

Every algorithm of the ladder is compared element by element with the oracle on
the same seeded inputs: bitwise where the exact result is representable (all-ones,
identity, small integers), within |C - C_oracle| <= 5e-4*S + 1e-6 otherwise.  The
workloads are the square 512^3 and 1024^3 products, the 2048 x 3072 x 4096
product, the ragged 4095 x 4097 x 1023 and 1 x 4096 x 4096 products, and the
8192^3 product; the largest ones are compared on sampled rows, columns and
elements that the oracle computes one by one.  Guard bands around C catch
writes outside the matrix, NaN-filled row padding catches reads outside it.
"""
import functools

import numpy as np
import pytest

import dense_fp32_matrix_f32_amd as sg
import oracle
from gpu_helpers import (Device, assert_close, assert_guards, check_full, check_sampled, inputs,
                         log, torch_cuda)

pytestmark = pytest.mark.gpu

LADDER = [sg.ALGO_NAIVE, sg.ALGO_LDS_TILED, sg.ALGO_VALU_REGBLOCK, sg.ALGO_MFMA, sg.ALGO_BF16X6,
          sg.ALGO_SKINNY, sg.ALGO_SKINNY_N, sg.ALGO_AUTO]
FAST = [sg.ALGO_VALU_REGBLOCK, sg.ALGO_MFMA, sg.ALGO_AUTO]
name = sg.sgemm_f32_algo_name


def _run(A, B, M, N, K, algo, **kw):
    log(f"[gpu] {name(algo)} M={M} N={N} K={K} lda={A.shape[1]} ldb={B.shape[1]} {kw}")
    d = Device(A, B, M, N, K, **kw)
    d.run(algo)
    C, guards = d.result()
    assert_guards(guards)
    return C


# ---------------------------------------------------------------- small shapes
SMALL = [(1, 1, 1), (1, 7, 3), (2, 3, 5), (7, 8, 9), (15, 16, 17), (16, 16, 16), (31, 33, 63),
         (33, 31, 65), (63, 65, 127), (64, 64, 64), (65, 63, 129), (127, 129, 15),
         (128, 128, 128), (129, 127, 257), (9, 300, 4), (300, 9, 31), (257, 513, 77)]


@pytest.mark.parametrize("algo", LADDER, ids=name)
@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(map(str, s)))
def test_small_shapes_exact_integers(shape, algo):
    M, N, K = shape
    A, B = inputs(M, N, K, "smallint", seed=100 + M + N + K)
    C = _run(A, B, M, N, K, algo)
    check_full(A, B, M, N, K, C, f"{name(algo)} {shape}", exact=True)


@pytest.mark.parametrize("algo", LADDER, ids=name)
@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(map(str, s)))
def test_small_shapes_normal(shape, algo):
    M, N, K = shape
    A, B = inputs(M, N, K, "normal", seed=200 + M + N + K)
    C = _run(A, B, M, N, K, algo)
    check_full(A, B, M, N, K, C, f"{name(algo)} {shape}")


@pytest.mark.parametrize("algo", LADDER, ids=name)
@pytest.mark.parametrize("offset", [0, 1, 3])
def test_padded_and_misaligned(algo, offset):
    """Row strides beyond the row length, 4-byte-only alignment, several tiles, ragged tails."""
    M, N, K = 300, 517, 259
    A, B = inputs(M, N, K, "uniform_pm1", seed=7, lda=K + 5, ldb=N + 3)
    C = _run(A, B, M, N, K, algo, ldc=N + 7, offset_elems=offset)
    check_full(A, B, M, N, K, C, f"{name(algo)} padded offset={offset}")
    A, B = inputs(M, N, K, "smallint", seed=8, lda=K + 1, ldb=N + 1)
    C = _run(A, B, M, N, K, algo, ldc=N + 1, offset_elems=offset)
    check_full(A, B, M, N, K, C, f"{name(algo)} padded int offset={offset}", exact=True)


# ---------------------------------------------------------------- 512^3 and 1024^3
@functools.lru_cache(maxsize=None)
def _square_case(n, seed):
    A, B = inputs(n, n, n, "normal", seed=seed)
    Cref, S = oracle.sgemm(A, B)
    return A, B, Cref, S


@pytest.mark.parametrize("algo", LADDER, ids=name)
@pytest.mark.parametrize("n,seed", [(512, 1), (1024, 2)])
def test_square_normal(n, seed, algo):
    A, B, Cref, S = _square_case(n, seed)
    C = _run(A, B, n, n, n, algo)
    assert_close(C, Cref, S, f"{name(algo)} {n}^3")


@pytest.mark.parametrize("algo", LADDER, ids=name)
@pytest.mark.parametrize("n", [512, 1024])
def test_square_all_ones(n, algo):
    """Page "GPU programming with C++ and CUDA", chapter 7: all-ones inputs give the width."""
    A, B = inputs(n, n, n, "ones", seed=0)
    C = _run(A, B, n, n, n, algo)
    assert np.all(C == np.float32(n)), f"{name(algo)}: all-ones {n}^3 is not exactly {n}"


@pytest.mark.parametrize("algo", LADDER, ids=name)
def test_identity_b_1024(algo):
    n = 1024
    A, _ = inputs(n, n, n, "normal", seed=2)
    B = np.eye(n, dtype=np.float32)
    C = _run(A, B, n, n, n, algo)
    assert np.array_equal(C, A), f"{name(algo)}: A·I != A bitwise"


# ---------------------------------------------------------------- 2048 x 3072 x 4096
@pytest.mark.parametrize("algo", FAST + [sg.ALGO_NAIVE, sg.ALGO_LDS_TILED], ids=name)
def test_2048x3072x4096(algo):
    M, N, K = 2048, 3072, 4096
    A, B = inputs(M, N, K, "normal", seed=3)
    C = _run(A, B, M, N, K, algo)
    check_sampled(A, B, M, N, K, C, f"{name(algo)} 2048x3072x4096", seed=3)


# ---------------------------------------------------------------- ragged 4095 x 4097 x 1023
@pytest.mark.parametrize("algo", LADDER[:5] + [sg.ALGO_AUTO], ids=name)
def test_ragged_4095x4097x1023(algo):
    M, N, K = 4095, 4097, 1023
    A, B = inputs(M, N, K, "uniform_pm1", seed=4)
    C = _run(A, B, M, N, K, algo)
    check_sampled(A, B, M, N, K, C, f"{name(algo)} ragged", seed=4)
    A, B = inputs(M, N, K, "smallint", seed=44)
    C = _run(A, B, M, N, K, algo)
    check_sampled(A, B, M, N, K, C, f"{name(algo)} ragged int", exact=True, seed=44)


# ---------------------------------------------------------------- 1 x 4096 x 4096
@pytest.mark.parametrize("algo", LADDER, ids=name)
def test_row_times_matrix_1x4096x4096(algo):
    M, N, K = 1, 4096, 4096
    A, B = inputs(M, N, K, "uniform_pm1", seed=5)
    C = _run(A, B, M, N, K, algo)
    check_full(A, B, M, N, K, C, f"{name(algo)} 1x4096x4096")
    A, B = inputs(M, N, K, "smallint", seed=55)
    C = _run(A, B, M, N, K, algo)
    check_full(A, B, M, N, K, C, f"{name(algo)} 1x4096x4096 int", exact=True)


# ---------------------------------------------------------------- 8192^3
@functools.lru_cache(maxsize=1)
def _inputs_8192():
    n = 8192
    return inputs(n, n, n, "normal", seed=6)


@pytest.mark.parametrize("algo", [sg.ALGO_AUTO, sg.ALGO_VALU_REGBLOCK, sg.ALGO_BF16X6,
                                  sg.ALGO_NAIVE, sg.ALGO_LDS_TILED], ids=name)
def test_8192_cubed(algo):
    n = 8192
    A, B = _inputs_8192()
    C = _run(A, B, n, n, n, algo)
    check_sampled(A, B, n, n, n, C, f"{name(algo)} 8192^3", seed=6)


# ---------------------------------------------------------------- degenerate cases
@pytest.mark.parametrize("algo", LADDER, ids=name)
def test_k_zero_writes_zeros(algo):
    M, N = 37, 70
    A = np.zeros((M, 1), np.float32)
    B = np.zeros((1, N), np.float32)
    d = Device(A, B, M, N, 0, fill=np.nan)
    d.K = 0
    d.lda, d.ldb = 1, N
    d.run(algo)
    C, guards = d.result()
    assert np.all(C == 0)
    assert np.all(np.isnan(guards))


@pytest.mark.parametrize("algo", LADDER, ids=name)
def test_empty_m_or_n_touches_nothing(algo):
    torch = torch_cuda()
    c = torch.full((64,), 3.0, device="cuda")
    a = torch.ones(64, device="cuda")
    s = torch.cuda.current_stream()
    assert sg.sgemm_f32_algo(0, 8, 8, a.data_ptr(), 8, a.data_ptr(), 8, c.data_ptr(), 8,
                             s.cuda_stream, algo) == 0
    assert sg.sgemm_f32_algo(8, 0, 8, a.data_ptr(), 8, a.data_ptr(), 1, c.data_ptr(), 1,
                             s.cuda_stream, algo) == 0
    s.synchronize()
    assert torch.all(c == 3.0)


@pytest.mark.parametrize("algo", LADDER, ids=name)
def test_c_is_never_read(algo):
    """beta = 0: a NaN-filled C must not leak into the result."""
    M, N, K = 130, 200, 50
    A, B = inputs(M, N, K, "normal", seed=9)
    d = Device(A, B, M, N, K, fill=np.nan)
    d.run(algo)
    C, guards = d.result()
    assert np.all(np.isfinite(C))
    assert np.all(np.isnan(guards))
    check_full(A, B, M, N, K, C, f"{name(algo)} NaN-filled C")


@pytest.mark.parametrize("algo", LADDER, ids=name)
def test_nan_stays_in_its_row_and_column(algo):
    M, N, K = 150, 140, 90
    A, B = inputs(M, N, K, "normal", seed=10)
    A[17, 33] = np.nan
    B[40, 101] = np.inf
    C = _run(A, B, M, N, K, algo)
    assert np.all(np.isnan(C[17]))
    other = np.delete(np.delete(C, 17, axis=0), 101, axis=1)
    assert np.all(np.isfinite(other))
    assert not np.any(np.isfinite(np.delete(C[:, 101], 17)))


@pytest.mark.parametrize("algo", FAST + [sg.ALGO_SKINNY, sg.ALGO_SKINNY_N, sg.ALGO_BF16X6],
                         ids=name)
def test_bitwise_reproducible(algo):
    M, N, K = 1000, 1100, 700
    A, B = inputs(M, N, K, "normal", seed=11)
    d = Device(A, B, M, N, K)
    d.run(algo)
    C1, _ = d.result()
    d.run(algo)
    C2, _ = d.result()
    assert np.array_equal(C1.view(np.uint32), C2.view(np.uint32))


def test_non_default_stream():
    torch = torch_cuda()
    M, N, K = 520, 260, 130
    A, B = inputs(M, N, K, "normal", seed=12)
    d = Device(A, B, M, N, K)
    s = torch.cuda.Stream()
    d.run(sg.ALGO_AUTO, stream=s)
    C, guards = d.result()
    assert_guards(guards)
    check_full(A, B, M, N, K, C, "side stream")


def test_torch_matmul_helper():
    torch = torch_cuda()
    A, B = inputs(333, 444, 222, "normal", seed=13)
    At = torch.from_numpy(A).cuda()
    Bt = torch.from_numpy(B).cuda()
    C = sg.matmul(At, Bt)
    torch.cuda.synchronize()
    check_full(A, B, 333, 444, 222, C.cpu().numpy(), "matmul helper")
    # a strided view passes its row stride as the leading dimension
    C2 = sg.matmul(At[:, :100], Bt[:100, :])
    torch.cuda.synchronize()
    check_full(np.ascontiguousarray(A[:, :100]), np.ascontiguousarray(B[:100]), 333, 444, 100,
               C2.cpu().numpy(), "view")


def test_torch_matmul_rejects_broadcast_views():
    """Expanded (stride-0) or overlapping views have no leading dimension the library
    could use; the helper raises before any launch and leaves out untouched."""
    torch = torch_cuda()
    M, N, K = 64, 48, 32
    row_a = torch.ones(1, K, device="cuda")
    row_b = torch.ones(1, N, device="cuda")
    A = torch.ones(M, K, device="cuda")
    B = torch.ones(K, N, device="cuda")
    out = torch.full((M, N), 5.0, device="cuda")
    for a, b, o in [(row_a.expand(M, K), B, out), (A, row_b.expand(K, N), out),
                    (A, B, torch.full((1, N), 5.0, device="cuda").expand(M, N)),
                    (A, torch.ones(K, 1, device="cuda").expand(K, N), out),
                    (A.as_strided((M, K), (K // 2, 1)), B, out)]:
        with pytest.raises(ValueError):
            sg.matmul(a, b, out=o)
    torch.cuda.synchronize()
    assert torch.all(out == 5.0)


# ---------------------------------------------------------------- few columns
FEW_COLS = [(4096, 1, 4096), (4095, 3, 1023), (1000, 8, 777), (33, 5, 4099), (4096, 9, 257),
            (17, 2, 1), (300, 7, 5), (513, 2, 1031)]


@pytest.mark.parametrize("algo", [sg.ALGO_SKINNY_N, sg.ALGO_AUTO], ids=name)
@pytest.mark.parametrize("shape", FEW_COLS, ids=lambda s: "x".join(map(str, s)))
def test_few_columns(shape, algo):
    M, N, K = shape
    A, B = inputs(M, N, K, "smallint", seed=300 + M + N + K)
    C = _run(A, B, M, N, K, algo)
    check_full(A, B, M, N, K, C, f"{name(algo)} {shape} int", exact=True)
    A, B = inputs(M, N, K, "normal", seed=400 + M + N + K, lda=K + 1)
    C = _run(A, B, M, N, K, algo, offset_elems=1)
    check_full(A, B, M, N, K, C, f"{name(algo)} {shape}")
    # padded rows of B (NaN in the padding): rows of B narrower than the kernel's
    # vectors are read whole, padding included, which must not reach C
    A, B = inputs(M, N, K, "normal", seed=500 + M + N + K, ldb=N + 3)
    C = _run(A, B, M, N, K, algo)
    check_full(A, B, M, N, K, C, f"{name(algo)} {shape} padded B")


# One or two columns of a wide B (rows of y at least a cache line apart): the
# few-columns kernel gathers y into LDS per work-group, in chunks of k, zero past
# K.  Several chunks with a partial last one, K not a multiple of 4, rows that do
# not fill the last work-group, NaN in B's padding.
WIDE_B = [(4095, 1, 1023, 4097), (777, 2, 2500, 64), (300, 1, 4099, 33), (1000, 2, 5000, 100),
          (33, 1, 256, 32), (5000, 2, 2049, 4096), (257, 1, 300, 40), (8193, 2, 1999, 48)]


@pytest.mark.parametrize("algo", [sg.ALGO_SKINNY_N, sg.ALGO_AUTO], ids=name)
@pytest.mark.parametrize("case", WIDE_B, ids=lambda c: "x".join(map(str, c[:3])) + f"-ldb{c[3]}")
def test_few_columns_of_wide_b(case, algo):
    M, N, K, ldb = case
    A, B = inputs(M, N, K, "smallint", seed=700 + M + K, ldb=ldb)
    C = _run(A, B, M, N, K, algo)
    check_full(A, B, M, N, K, C, f"{name(algo)} {case} int", exact=True)
    A, B = inputs(M, N, K, "normal", seed=800 + M + K, lda=K + 3, ldb=ldb)
    C = _run(A, B, M, N, K, algo, offset_elems=1)
    check_full(A, B, M, N, K, C, f"{name(algo)} {case}")


# ---------------------------------------------------------------- 64-bit offsets
def _big_case(M, N, K, algo, rows=None, cols=None):
    """An operand of more than 2^31 elements, drawn on the device (seeded); the
    oracle checks whole sampled rows and columns of C from host copies of the
    rows of A and columns of B they need."""
    torch = torch_cuda()
    gen = torch.Generator(device="cuda")
    gen.manual_seed(77)
    dA = torch.empty((M, K), device="cuda").uniform_(-1, 1, generator=gen)
    dB = torch.empty((K, N), device="cuda").uniform_(-1, 1, generator=gen)
    dC = torch.full((M, N), float("nan"), device="cuda")
    log(f"[gpu] 64-bit offsets {name(algo)} M={M} N={N} K={K}")
    st = sg.sgemm_f32_algo(M, N, K, dA.data_ptr(), K, dB.data_ptr(), N, dC.data_ptr(), N,
                           torch.cuda.current_stream().cuda_stream, algo)
    assert st == 0
    torch.cuda.synchronize()
    rows = rows if rows is not None else [0, 1, M // 2, M - 2, M - 1]
    cols = cols if cols is not None else [0, 1, N // 2, N - 2, N - 1]
    rows = sorted(set(r for r in rows if 0 <= r < M))
    cols = sorted(set(c for c in cols if 0 <= c < N))
    Bh = dB[:, cols].cpu().numpy()
    Ar = dA[rows].cpu().numpy()
    Cref, S = oracle.sgemm(np.ascontiguousarray(Ar), np.ascontiguousarray(Bh))
    Cg = dC[rows][:, cols].cpu().numpy()
    assert_close(Cg, Cref, S, f"{name(algo)} rows x cols beyond 2^31 elements")
    del dA, dB, dC
    torch.cuda.empty_cache()


def test_offsets_beyond_2_31_mfma():
    # A: 131073 x 16387 = 2.148e9 elements; its last rows start past 2^31.
    _big_case(131073, 40, 16387, sg.ALGO_AUTO)


def test_offsets_beyond_2_31_few_columns():
    _big_case(131073, 3, 16387, sg.ALGO_SKINNY_N)


def test_offsets_beyond_2_31_few_rows():
    # B: 65537 x 32769 = 2.148e9 elements; its last rows start past 2^31.
    _big_case(3, 32769, 65537, sg.ALGO_SKINNY)

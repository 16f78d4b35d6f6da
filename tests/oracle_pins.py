"""Pins for the CPU oracle: facts fixed by the pages or by mathematics.

Each ``pin_*`` takes an oracle library handle (``oracle.load(path)``) and raises
AssertionError if the oracle disagrees with the fact.  The pins are shared by
``test_oracle_pins.py`` (the real oracle must pass all of them) and
``test_oracle_mutants.py`` (every oracle with a planted mistake must fail at
least one of them).
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np

import oracle
import synthgen

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_golden(name: str) -> dict:
    """Parse a ``key = value`` fixture (``#`` starts a comment)."""
    out = {}
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if "=" in line:
                k, v = line.split("=", 1)
                out[k.strip()] = v.strip()
    return out


def read_golden_rows(name: str) -> list[list[int]]:
    rows = []
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append([int(t) for t in line.split()])
    return rows


def _gen(rows, cols, seed, stream, dist, ld=None):
    return synthgen.matrix(rows, cols, seed=seed, stream=stream, dist=dist, ld=ld)[:, :cols]


def pin_all_ones(lib):
    """All-ones A and B give C = K and S = K at every element (page "GPU programming
    with C++ and CUDA", chapter 7, examples 1 and 2 check the width)."""
    for M, N, K in read_golden_rows("all_ones.txt"):
        if M * N * K > 40_000_000:
            # the 1024^3 case: check a band of rows through the listed-element path
            A = synthgen.ones(M, K)
            B = synthgen.ones(K, N)
            r = np.repeat(np.array([0, M // 2, M - 1]), N)
            c = np.tile(np.arange(N), 3)
            C, S = oracle.sgemm_elems(A, B, r, c, lib=lib)
        else:
            C, S = oracle.sgemm(synthgen.ones(M, K), synthgen.ones(K, N), lib=lib)
        assert np.all(C == K), f"all-ones {M}x{N}x{K}: C != K"
        assert np.all(S == K), f"all-ones {M}x{N}x{K}: S != K"


def pin_identity(lib):
    """A·I = A and I·B = B exactly: one nonzero term per element."""
    A = _gen(37, 29, 11, 0, "normal")
    C, S = oracle.sgemm(A, synthgen.identity(29), lib=lib)
    assert np.array_equal(C, A.astype(np.float64)), "A·I != A"
    assert np.array_equal(S, np.abs(A).astype(np.float64)), "S(A·I) != |A|"
    B = _gen(23, 41, 11, 1, "normal")
    C, _ = oracle.sgemm(synthgen.identity(23), B, lib=lib)
    assert np.array_equal(C, B.astype(np.float64)), "I·B != B"


def pin_small_integers(lib):
    """Integer entries in [-4, 4]: every partial sum is an exact integer, so C equals
    the exact integer product (computed here with Python/numpy int64)."""
    for (M, N, K) in [(5, 7, 3), (17, 13, 31), (1, 65, 40), (33, 1, 70)]:
        A = _gen(M, K, 21, 0, "smallint")
        B = _gen(K, N, 21, 1, "smallint")
        exact = A.astype(np.int64) @ B.astype(np.int64)
        C, S = oracle.sgemm(A, B, lib=lib)
        assert np.array_equal(C, exact.astype(np.float64)), f"small-int {M}x{N}x{K}"
        sabs = np.abs(A).astype(np.int64) @ np.abs(B).astype(np.int64)
        assert np.array_equal(S, sabs.astype(np.float64)), f"small-int S {M}x{N}x{K}"


def pin_block_identity(lib):
    """The 8x8 / TILE 4 worked example of the page "【infra之路】Tiled Matrix
    Multiplication详解": C00 = A00·B00 + A01·B10 (exact on integer data)."""
    g = read_golden("tiled_block_example.txt")
    n, t = int(g["n"]), int(g["tile"])
    A = _gen(n, n, 31, 0, "smallint")
    B = _gen(n, n, 31, 1, "smallint")
    C, _ = oracle.sgemm(A, B, lib=lib)
    A00, A01 = np.ascontiguousarray(A[:t, :t]), np.ascontiguousarray(A[:t, t:])
    B00, B10 = np.ascontiguousarray(B[:t, :t]), np.ascontiguousarray(B[t:, :t])
    P0, _ = oracle.sgemm(A00, B00, lib=lib)
    P1, _ = oracle.sgemm(A01, B10, lib=lib)
    assert np.array_equal(C[:t, :t], P0 + P1), "C00 != A00·B00 + A01·B10"
    # and every other block, as the same statement for (bi, bj)
    for bi in range(n // t):
        for bj in range(n // t):
            acc = np.zeros((t, t))
            for bk in range(n // t):
                Ab = np.ascontiguousarray(A[bi * t:(bi + 1) * t, bk * t:(bk + 1) * t])
                Bb = np.ascontiguousarray(B[bk * t:(bk + 1) * t, bj * t:(bj + 1) * t])
                acc += oracle.sgemm(Ab, Bb, lib=lib)[0]
            assert np.array_equal(C[bi * t:(bi + 1) * t, bj * t:(bj + 1) * t], acc)


def pin_transpose(lib):
    """(A·B)^T = B^T·A^T, bitwise: each element sums the same products in the same
    k order."""
    A = _gen(19, 27, 41, 0, "normal")
    B = _gen(27, 12, 41, 1, "normal")
    C, S = oracle.sgemm(A, B, lib=lib)
    Ct, St = oracle.sgemm(np.ascontiguousarray(B.T), np.ascontiguousarray(A.T), lib=lib)
    assert np.array_equal(C.T, Ct), "(AB)^T != B^T A^T"
    assert np.array_equal(S.T, St)


def _fraction_product(A, B, i, j):
    return sum((Fraction(float(A[i, k])) * Fraction(float(B[k, j])) for k in range(A.shape[1])),
               Fraction(0))


def pin_brute_force(lib):
    """Tiny shapes against an exact rational sum: the fp64 running sum of exact
    products is within K·2^-53·S of the true value (recursive summation bound)."""
    for (M, N, K, dist) in [(3, 4, 5, "normal"), (6, 2, 9, "uniform_pm1"), (1, 1, 17, "normal"),
                            (4, 3, 1, "normal")]:
        A = _gen(M, K, 51, 0, dist)
        B = _gen(K, N, 51, 1, dist)
        C, S = oracle.sgemm(A, B, lib=lib)
        for i in range(M):
            for j in range(N):
                exact = _fraction_product(A, B, i, j)
                s_exact = sum((abs(Fraction(float(A[i, k]))) * abs(Fraction(float(B[k, j])))
                               for k in range(K)), Fraction(0))
                bound = K * 2.0 ** -53 * float(s_exact) * 1.0001
                assert abs(Fraction(C[i, j]) - exact) <= Fraction(bound), (M, N, K, i, j)
                assert abs(Fraction(S[i, j]) - s_exact) <= Fraction(bound), (M, N, K, i, j)
                assert math.isclose(S[i, j], float(s_exact), rel_tol=1e-14)


def pin_library_fp64(lib):
    """Against numpy's float64 matmul (an independent routine), within the fp64
    summation bound of both sides."""
    A = _gen(45, 70, 61, 0, "normal")
    B = _gen(70, 38, 61, 1, "normal")
    C, S = oracle.sgemm(A, B, lib=lib)
    ref = A.astype(np.float64) @ B.astype(np.float64)
    sref = np.abs(A).astype(np.float64) @ np.abs(B).astype(np.float64)
    tol = 2 * 70 * 2.0 ** -53 * sref
    assert np.all(np.abs(C - ref) <= tol)
    assert np.all(np.abs(S - sref) <= tol)


def pin_elements_match_full(lib):
    """Listed elements are bit-identical to the same elements of the full product."""
    M, N, K = 23, 31, 57
    A = _gen(M, K, 71, 0, "normal")
    B = _gen(K, N, 71, 1, "normal")
    C, S = oracle.sgemm(A, B, lib=lib)
    rng = np.random.default_rng(5)
    r = rng.integers(0, M, 200)
    c = rng.integers(0, N, 200)
    Ce, Se = oracle.sgemm_elems(A, B, r, c, lib=lib)
    assert np.array_equal(Ce, C[r, c]) and np.array_equal(Se, S[r, c])


def pin_leading_dimensions(lib):
    """Row padding (filled with NaN) is never read: padded operands give the dense
    operands' result."""
    M, N, K = 9, 14, 21
    Ap = synthgen.matrix(M, K, seed=81, stream=0, dist="normal", ld=K + 5)
    Bp = synthgen.matrix(K, N, seed=81, stream=1, dist="normal", ld=N + 3)
    C1, S1 = oracle.sgemm(Ap[:, :K], Bp[:, :N], lib=lib)
    C2, S2 = oracle.sgemm(np.ascontiguousarray(Ap[:, :K]), np.ascontiguousarray(Bp[:, :N]),
                          lib=lib)
    assert np.all(np.isfinite(C1))
    assert np.array_equal(C1, C2) and np.array_equal(S1, S2)


def pin_empty_sum(lib):
    """K = 0 is the empty sum: C = 0, S = 0."""
    A = np.zeros((4, 0), dtype=np.float32)
    B = np.zeros((0, 6), dtype=np.float32)
    C, S = oracle.sgemm(A, B, lib=lib)
    assert C.shape == (4, 6) and np.all(C == 0) and np.all(S == 0)


# ---- the general form: alpha * op(A) op(B) + beta * C ----

def _stored(X, trans):
    """The array that holds X (M x K) when it is passed transposed or not."""
    return np.ascontiguousarray(X.T) if trans else X


def pin_ex_brute_force(lib):
    """Tiny shapes, all four operand layouts, several alpha/beta, against exact
    rational arithmetic: alpha*sum + beta*c in Fractions, within the fp64
    summation bound (K + 2 roundings of the scale)."""
    cases = [(3, 4, 5, 1.0, 0.0), (2, 5, 3, -0.5, 1.0), (4, 3, 6, 3.0, -2.25), (1, 1, 7, 0.75, 0.5)]
    for n, (M, N, K, alpha, beta) in enumerate(cases):
        X = _gen(M, K, 90 + n, 0, "normal")       # op(A)
        Y = _gen(K, N, 90 + n, 1, "normal")       # op(B)
        Cin = _gen(M, N, 90 + n, 2, "normal")
        for ta in (False, True):
            for tb in (False, True):
                C, S = oracle.sgemm_ex(_stored(X, ta), _stored(Y, tb), ta, tb, alpha, beta, Cin,
                                       lib=lib)
                for i in range(M):
                    for j in range(N):
                        prod = _fraction_product(X, Y, i, j)
                        sabs = sum((abs(Fraction(float(X[i, k]))) * abs(Fraction(float(Y[k, j])))
                                    for k in range(K)), Fraction(0))
                        exact = Fraction(alpha) * prod + Fraction(beta) * Fraction(float(Cin[i, j]))
                        s_exact = (abs(Fraction(alpha)) * sabs +
                                   abs(Fraction(beta)) * abs(Fraction(float(Cin[i, j]))))
                        bound = Fraction((K + 2) * 2.0 ** -53 * float(s_exact) * 1.0001)
                        assert abs(Fraction(C[i, j]) - exact) <= bound, (ta, tb, M, N, K, i, j)
                        assert abs(Fraction(S[i, j]) - s_exact) <= bound, (ta, tb, i, j)


def pin_ex_library_fp64(lib):
    """All four layouts against numpy's float64 matmul of the explicit transposes."""
    M, N, K = 37, 29, 53
    X = _gen(M, K, 95, 0, "normal")
    Y = _gen(K, N, 95, 1, "normal")
    Cin = _gen(M, N, 95, 2, "uniform_pm1")
    alpha, beta = -1.25, 0.375
    ref = alpha * (X.astype(np.float64) @ Y.astype(np.float64)) + beta * Cin.astype(np.float64)
    sref = (abs(alpha) * (np.abs(X).astype(np.float64) @ np.abs(Y).astype(np.float64)) +
            abs(beta) * np.abs(Cin).astype(np.float64))
    tol = 2 * (K + 2) * 2.0 ** -53 * sref
    for ta in (False, True):
        for tb in (False, True):
            C, S = oracle.sgemm_ex(_stored(X, ta), _stored(Y, tb), ta, tb, alpha, beta, Cin,
                                   lib=lib)
            assert np.all(np.abs(C - ref) <= tol), (ta, tb)
            assert np.all(np.abs(S - sref) <= tol), (ta, tb)
            r = np.array([0, M - 1, 5, 17])
            c = np.array([N - 1, 0, 3, 28])
            Ce, Se = oracle.sgemm_ex(_stored(X, ta), _stored(Y, tb), ta, tb, alpha, beta, Cin,
                                     rows=r, cols=c, lib=lib)
            assert np.array_equal(Ce, C[r, c]) and np.array_equal(Se, S[r, c]), (ta, tb)


def pin_ex_plain_form(lib):
    """alpha = 1, beta = 0 with untransposed operands is the plain product, bitwise
    (same k order), and a transposed store of the same operand gives the same bits."""
    X = _gen(21, 33, 97, 0, "normal")
    Y = _gen(33, 18, 97, 1, "normal")
    C0, S0 = oracle.sgemm(X, Y, lib=lib)
    zero_c = np.zeros((21, 18), dtype=np.float32)
    for ta in (False, True):
        for tb in (False, True):
            C, S = oracle.sgemm_ex(_stored(X, ta), _stored(Y, tb), ta, tb, C=zero_c, lib=lib)
            assert np.array_equal(C, C0) and np.array_equal(S, S0), (ta, tb)


def pin_ex_closed_forms(lib):
    """All-ones operands: C = alpha*K + beta*c exactly; beta == 0 never reads C (NaN
    there stays out); alpha == 0 never reads A or B (NaN there stays out); a second
    call with beta = -1 and C = the first result cancels to 0 on integer data."""
    M, N, K = 6, 7, 12
    ones_a, ones_b = synthgen.ones(M, K), synthgen.ones(K, N)
    Cin = np.full((M, N), 3.0, dtype=np.float32)
    C, S = oracle.sgemm_ex(ones_a, ones_b, alpha=2.0, beta=-0.5, C=Cin, lib=lib)
    assert np.all(C == 2.0 * K - 1.5) and np.all(S == 2.0 * K + 1.5)
    nan_c = np.full((M, N), np.nan, dtype=np.float32)
    C, S = oracle.sgemm_ex(ones_a, ones_b, alpha=1.5, beta=0.0, C=nan_c, lib=lib)
    assert np.all(C == 1.5 * K) and np.all(S == 1.5 * K)
    nan_a = np.full((M, K), np.nan, dtype=np.float32)
    nan_b = np.full((K, N), np.nan, dtype=np.float32)
    C, S = oracle.sgemm_ex(nan_a, nan_b, alpha=0.0, beta=1.5, C=Cin, lib=lib)
    assert np.all(C == 4.5) and np.all(S == 4.5)
    A = _gen(M, K, 99, 0, "smallint")
    B = _gen(K, N, 99, 1, "smallint")
    P = (A.astype(np.int64) @ B.astype(np.int64)).astype(np.float32)
    C, _ = oracle.sgemm_ex(A, B, alpha=1.0, beta=-1.0, C=P, lib=lib)
    assert np.all(C == 0.0)


def _padded_store(X, trans, pad):
    """The stored array of the logical operand X, transposed or not, as a view with
    ``pad`` NaN floats at the end of every stored row (so ld = row length + pad)."""
    st = X.T if trans else X
    r, c = st.shape
    buf = np.full((r, c + pad), np.nan, dtype=np.float32)
    buf[:, :c] = st
    return buf[:, :c]


def pin_ex_padded_strides(lib):
    """Padded leading dimensions in all four layouts and for C_in, against the exact
    integer result: alpha*sum_k opA[i][k]*opB[k][j] + beta*C_in[i][j] (the definition
    of page "CUDA算子优化(4)：矩阵乘法", section "矩阵乘法的数学定义", with the BLAS
    operands).  Every stored row carries NaN padding, and M, N, K and the three
    paddings all differ, so reading any array with a row length in place of its
    leading dimension (or a padding element) gives a wrong or non-finite value."""
    M, N, K = 7, 9, 11
    X = _gen(M, K, 101, 0, "smallint")      # op(A)
    Y = _gen(K, N, 101, 1, "smallint")      # op(B)
    Cin = _gen(M, N, 101, 2, "smallint")
    alpha, beta = 2, -3
    xi, yi, ci = X.astype(np.int64), Y.astype(np.int64), Cin.astype(np.int64)
    exact = (alpha * (xi @ yi) + beta * ci).astype(np.float64)
    sabs = (abs(alpha) * (np.abs(xi) @ np.abs(yi)) + abs(beta) * np.abs(ci)).astype(np.float64)
    Cp = _padded_store(Cin, False, 4)
    assert Cp.strides[0] == 4 * (N + 4)
    rng = np.random.default_rng(9)
    r = rng.integers(0, M, 40)
    c = rng.integers(0, N, 40)
    for ta in (False, True):
        for tb in (False, True):
            A = _padded_store(X, ta, 3)
            B = _padded_store(Y, tb, 5)
            C, S = oracle.sgemm_ex(A, B, ta, tb, float(alpha), float(beta), Cp, lib=lib)
            assert np.array_equal(C, exact), ("padded strides", ta, tb)
            assert np.array_equal(S, sabs), ("padded strides S", ta, tb)
            Ce, Se = oracle.sgemm_ex(A, B, ta, tb, float(alpha), float(beta), Cp, rows=r,
                                     cols=c, lib=lib)
            assert np.array_equal(Ce, exact[r, c]) and np.array_equal(Se, sabs[r, c]), (ta, tb)


ALL_PINS = [pin_all_ones, pin_identity, pin_small_integers, pin_block_identity,
            pin_transpose, pin_brute_force, pin_library_fp64, pin_elements_match_full,
            pin_leading_dimensions, pin_empty_sum, pin_ex_brute_force, pin_ex_library_fp64,
            pin_ex_plain_form, pin_ex_closed_forms, pin_ex_padded_strides]

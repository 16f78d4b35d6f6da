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


ALL_PINS = [pin_all_ones, pin_identity, pin_small_integers, pin_block_identity,
            pin_transpose, pin_brute_force, pin_library_fp64, pin_elements_match_full,
            pin_leading_dimensions, pin_empty_sum]

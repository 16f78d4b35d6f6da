"""The blocked host SGEMM baseline against the oracle: it is only a timing
baseline, but its results must still be a correct product."""
import numpy as np
import pytest

import hostsgemm
import oracle
import synthgen


@pytest.mark.parametrize("shape", [(1, 1, 1), (1, 4096, 300), (300, 1, 77), (7, 17, 5),
                                   (97, 203, 259), (130, 2050, 513), (6, 16, 256)],
                         ids=lambda s: "x".join(map(str, s)))
def test_matches_oracle(shape):
    M, N, K = shape
    A = synthgen.matrix(M, K, seed=70, stream=0, dist="normal")
    B = synthgen.matrix(K, N, seed=70, stream=1, dist="normal")
    C = hostsgemm.sgemm(A, B, threads=3)
    R, S = oracle.sgemm(A, B)
    assert oracle.accept(C, R, S)


def test_exact_on_small_integers_and_padded_views():
    M, N, K = 53, 71, 300
    A = synthgen.matrix(M, K, seed=71, stream=0, dist="smallint", ld=K + 3)[:, :K]
    B = synthgen.matrix(K, N, seed=71, stream=1, dist="smallint", ld=N + 5)[:, :N]
    C = hostsgemm.sgemm(A, B, threads=4)
    exact = A.astype(np.int64) @ B.astype(np.int64)
    assert np.array_equal(C.astype(np.int64), exact)


def test_empty_sum_and_threads_beyond_rows():
    A = np.zeros((4, 0), dtype=np.float32)
    B = np.zeros((0, 5), dtype=np.float32)
    assert np.all(hostsgemm.sgemm(A, B) == 0)
    A = synthgen.matrix(2, 9, seed=72, stream=0, dist="smallint")
    B = synthgen.matrix(9, 3, seed=72, stream=1, dist="smallint")
    C = hostsgemm.sgemm(A, B, threads=64)
    assert np.array_equal(C.astype(np.int64), A.astype(np.int64) @ B.astype(np.int64))

"""Seeded random cases of the general form against the oracle: ragged shapes from
1 to 3000 (k to 9000), every storage order, padded leading dimensions with NaN
in the padding, integer alpha and beta, the automatic choice and forced rungs and
tile configurations.  Small-integer inputs keep every partial sum below 2^24, so
every correct summation order gives the exact result and the comparison is
bitwise (on sampled elements for the largest cases).  Eight chunks of 60 cases,
each case logged before it runs.
"""
import random

import pytest

import dense_fp32_matrix_f32_amd as sg
import synthgen
from gpu_helpers import Device, assert_guards, check_ex, log, sample_indices, stored

pytestmark = pytest.mark.gpu

CHUNKS, PER_CHUNK = 8, 60


def _dim(rng):
    r = rng.random()
    if r < 0.25:
        return rng.randint(1, 9)
    if r < 0.6:
        return rng.randint(10, 300)
    if r < 0.9:
        return rng.randint(300, 1500)
    return rng.randint(1500, 3000)


def _case(rng, ntiles):
    M, N, K = _dim(rng), _dim(rng), _dim(rng)
    if rng.random() < 0.15:
        K = rng.randint(1000, 9000)
    ta, tb = rng.randint(0, 1), rng.randint(0, 1)
    pad_a = rng.choice([0, 0, 0, 1, 3, 40])
    pad_b = rng.choice([0, 0, 0, 2, 5, 64])
    alpha = float(rng.choice([1, 1, 2, -1, 3]))
    beta = float(rng.choice([0, 0, 1, -2]))
    algo = rng.choice([sg.ALGO_AUTO] * 6 + [sg.ALGO_MFMA, sg.ALGO_SKINNY, sg.ALGO_SKINNY_N,
                                            sg.ALGO_NAIVE, sg.ALGO_LDS_TILED])
    if (algo == sg.ALGO_SKINNY and M > 8) or (algo == sg.ALGO_SKINNY_N and N > 8):
        algo = sg.ALGO_AUTO
    if algo in (sg.ALGO_NAIVE, sg.ALGO_LDS_TILED) and M * N * K > 2e9:
        algo = sg.ALGO_AUTO
    tile = rng.randrange(ntiles) if algo == sg.ALGO_MFMA and rng.random() < 0.6 else None
    return M, N, K, ta, tb, pad_a, pad_b, alpha, beta, algo, tile, rng.randrange(1 << 30)


@pytest.mark.parametrize("chunk", range(CHUNKS))
def test_random_general_form_exact(chunk):
    rng = random.Random(2024 + chunk)
    ntiles = sg.sgemm_f32_mfma_tiles()
    for i in range(PER_CHUNK):
        M, N, K, ta, tb, pad_a, pad_b, alpha, beta, algo, tile, seed = _case(rng, ntiles)
        X = synthgen.matrix(M, K, seed=seed, stream=0, dist="smallint")   # op(A)
        Y = synthgen.matrix(K, N, seed=seed, stream=1, dist="smallint")   # op(B)
        C0 = synthgen.matrix(M, N, seed=seed, stream=2, dist="smallint")
        As = stored(X, ta, (M if ta else K) + pad_a if pad_a else None)
        Bs = stored(Y, tb, (K if tb else N) + pad_b if pad_b else None)
        what = (f"chunk {chunk} case {i}: M={M} N={N} K={K} {'T' if ta else 'N'}"
                f"{'T' if tb else 'N'} pads {pad_a},{pad_b} alpha={alpha} beta={beta} "
                f"{sg.sgemm_f32_algo_name(algo)} tile={tile}")
        log(f"[gpu] {what}")
        d = Device(As, Bs, M, N, K, c_init=C0)
        d.run_ex(ta, tb, alpha, beta, algo=algo, tile=tile)
        C, guards = d.result()
        assert_guards(guards)
        rows = cols = None
        if M * N * K > 3e8:
            rows, cols = sample_indices(M, N, rows=3, cols=3, elems=1024, seed=i)
        check_ex(As, Bs, M, N, K, ta, tb, alpha, beta, C0, C, what, exact=True, rows=rows,
                 cols=cols)

"""A product whose C has more than 2^31 elements (46401 x 46403, 8.6 GB, both
ragged for every block size): every element offset past 2^31 must be formed in
64 bits on every rung.  Small-integer inputs make every summation order exact,
so the rows checked (the first, the rows around element 2^31 and the last) are
compared bitwise with the oracle; a guard band after C must stay untouched.
"""
import numpy as np
import pytest

import dense_fp32_matrix_f32_amd as sg
import oracle
import synthgen
from gpu_helpers import SENTINEL, log

pytestmark = pytest.mark.gpu

M, N = 46401, 46403    # M * N = 2,153,145,203 > 2^31
K = 9
GUARD = 4096
CROSS = (1 << 31) // N  # the row holding element 2^31
ROWS = [0, CROSS - 1, CROSS, CROSS + 1, M - 2, M - 1]


@pytest.fixture(scope="module")
def big():
    import torch
    assert M * N > 1 << 31
    X = synthgen.matrix(M, K, seed=91, stream=0, dist="smallint")
    Y = synthgen.matrix(K, N, seed=91, stream=1, dist="smallint")
    exact, _ = oracle.sgemm(np.ascontiguousarray(X[ROWS]), Y)
    dA = torch.from_numpy(X).cuda()
    dB = torch.from_numpy(Y).cuda()
    dC = torch.empty(M * N + GUARD, dtype=torch.float32, device="cuda")
    yield X, Y, exact, dA, dB, dC
    del dA, dB, dC
    torch.cuda.empty_cache()


def _check(dC, expect, what):
    import torch
    torch.cuda.synchronize()
    got = np.stack([dC[r * N:(r + 1) * N].cpu().numpy() for r in ROWS]).astype(np.float64)
    bad = np.argwhere(got != expect)
    assert bad.size == 0, f"{what}: {len(bad)} wrong, first at row {ROWS[bad[0][0]]} col {bad[0][1]}"
    guard = dC[M * N:].cpu().numpy()
    assert np.all(guard.view(np.uint32) == SENTINEL.view(np.uint32)), f"{what}: wrote past C"


RUNS = [("auto", None), ("naive", None), ("lds_tiled", None), ("valu_regblock", None),
        ("bf16x6", None)] + [("mfma", t) for t in range(sg.sgemm_f32_mfma_tiles())]


@pytest.mark.parametrize("run", RUNS, ids=lambda r: r[0] if r[1] is None else f"tile{r[1]}")
def test_c_past_2_31_elements(big, run):
    import torch
    X, Y, exact, dA, dB, dC = big
    algo, tile = run
    s = torch.cuda.current_stream().cuda_stream
    dC[:M * N].fill_(float("nan"))   # beta = 0: C is never read
    dC[M * N:].fill_(float(SENTINEL))
    log(f"[gpu] C past 2^31 elements: {algo} tile={tile} M={M} N={N} K={K}")
    if tile is None:
        st = sg.sgemm_f32_algo(M, N, K, dA.data_ptr(), K, dB.data_ptr(), N, dC.data_ptr(), N, s,
                               sg.ALGOS[algo])
    else:
        st = sg.sgemm_f32_mfma_tile(M, N, K, dA.data_ptr(), K, dB.data_ptr(), N, dC.data_ptr(), N,
                                    s, tile)
    assert st == 0
    _check(dC, exact, f"{algo} tile {tile}")


def test_c_past_2_31_elements_alpha_beta_and_k_zero(big):
    """The general form reads C (beta != 0) past 2^31 elements; with K = 0 the
    whole of C is scaled without a product."""
    import torch
    X, Y, exact, dA, dB, dC = big
    s = torch.cuda.current_stream().cuda_stream
    dC[:M * N].fill_(3.0)
    dC[M * N:].fill_(float(SENTINEL))
    log(f"[gpu] C past 2^31 elements: general form alpha=2 beta=-1 M={M} N={N} K={K}")
    st = sg.sgemm_f32_ex(0, 0, M, N, K, 2.0, dA.data_ptr(), K, dB.data_ptr(), N, -1.0,
                         dC.data_ptr(), N, s)
    assert st == 0
    _check(dC, 2.0 * exact - 3.0, "alpha 2 beta -1")
    log(f"[gpu] C past 2^31 elements: K=0 beta=0.5 M={M} N={N}")
    st = sg.sgemm_f32_ex(0, 0, M, N, 0, 1.0, dA.data_ptr(), 1, dB.data_ptr(), N, 0.5,
                         dC.data_ptr(), N, s)
    assert st == 0
    _check(dC, 0.5 * (2.0 * exact - 3.0), "K = 0, beta 0.5")

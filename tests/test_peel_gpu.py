"""Products that the automatic choice splits into a block part and an edge strip
(N or M lying 1 to 8 past a multiple of 32), against the oracle through the C ABI:
every storage order, small-integer data compared bitwise (with integer alpha and
beta), N(0,1) data within the tolerance, and guard bands around C.  Every element
of each strip is compared, plus whole rows and columns and random elements of the
block part."""
import numpy as np
import pytest

import dense_fp32_matrix_f32_amd as sg
import synthgen
from gpu_helpers import Device, assert_guards, check_ex, log, sample_indices, stored

pytestmark = pytest.mark.gpu

N_, T_ = sg.OP_N, sg.OP_T
LAYOUTS = [(N_, N_), (N_, T_), (T_, N_), (T_, T_)]
lid = lambda l: ("T" if l[0] else "N") + ("T" if l[1] else "N")

# (M, N, K): a column strip (4095 x 4097 x 1023, the ragged workload), a row strip,
# and both at once.
SHAPES = [(4095, 4097, 1023), (4097, 4095, 1023), (2049, 4097, 1023)]


def _split(M, N, K, ta, tb):
    torch = __import__("torch")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    algo, m_main, n_main = sg.sgemm_f32_auto_plan(ta, tb, M, N, K, cus)
    assert algo == sg.ALGO_MFMA
    return m_main, n_main


def _elements(M, N, m_main, n_main, seed):
    r, c = sample_indices(M, N, rows=6, cols=6, elems=4096, seed=seed)
    rows, cols = [r], [c]
    if n_main < N:   # the column strip: columns [n_main, N) of every row
        rows.append(np.repeat(np.arange(M), N - n_main))
        cols.append(np.tile(np.arange(n_main, N), M))
    if m_main < M:   # the row strip: rows [m_main, M) of columns [0, n_main)
        rows.append(np.repeat(np.arange(m_main, M), n_main))
        cols.append(np.tile(np.arange(n_main), M - m_main))
    # the first block row and column next to the strips
    rows.append(np.repeat(np.arange(max(m_main - 2, 0), m_main), N))
    cols.append(np.tile(np.arange(N), min(2, m_main)))
    return np.concatenate(rows), np.concatenate(cols)


@pytest.mark.parametrize("layout", LAYOUTS, ids=lid)
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("dist", ["smallint", "normal"])
def test_auto_split(shape, layout, dist):
    M, N, K = shape
    ta, tb = layout
    m_main, n_main = _split(M, N, K, ta, tb)
    assert (m_main, n_main) != (M, N), "the cost model no longer splits this shape"
    assert M - m_main <= 8 and N - n_main <= 8
    seed = 700 + M % 97 + N % 89
    X = synthgen.matrix(M, K, seed=seed, stream=0, dist=dist)
    Y = synthgen.matrix(K, N, seed=seed, stream=1, dist=dist)
    C0 = synthgen.matrix(M, N, seed=seed, stream=2, dist="smallint")
    As, Bs = stored(X, ta), stored(Y, tb)
    alpha, beta = (3.0, -2.0) if dist == "smallint" else (1.0, 0.0)
    log(f"[gpu] auto split {lid(layout)} {dist} M={M} N={N} K={K} main={m_main}x{n_main}")
    d = Device(As, Bs, M, N, K, c_init=C0)
    d.run_ex(ta, tb, alpha, beta)
    C, guards = d.result()
    assert_guards(guards)
    rows, cols = _elements(M, N, m_main, n_main, seed)
    check_ex(As, Bs, M, N, K, ta, tb, alpha, beta, C0, C,
             f"auto split {lid(layout)} {dist}", exact=dist == "smallint", rows=rows, cols=cols)

"""The general form C = alpha*op(A)*op(B) + beta*C against the oracle, through the
C ABI: every storage order of the operands on every rung that takes it, every
tile configuration of the matrix-core rung, alpha/beta scaling on the rungs that
only take untransposed operands, the product-free cases, C left unread when
beta == 0, and the column-major entry point.  Small-integer inputs with integer
alpha and beta make every correct summation order exact, so those cases are
compared bitwise.
"""
import numpy as np
import pytest

import dense_fp32_matrix_f32_amd as sg
import synthgen
from gpu_helpers import Device, assert_guards, check_ex, log, stored

pytestmark = pytest.mark.gpu

N_, T_ = sg.OP_N, sg.OP_T
LAYOUTS = [(N_, N_), (N_, T_), (T_, N_), (T_, T_)]
TRANS_ALGOS = [sg.ALGO_AUTO, sg.ALGO_NAIVE, sg.ALGO_LDS_TILED, sg.ALGO_MFMA, sg.ALGO_SKINNY,
               sg.ALGO_SKINNY_N]
NN_ONLY = [sg.ALGO_VALU_REGBLOCK, sg.ALGO_BF16X6]
lid = lambda l: ("T" if l[0] else "N") + ("T" if l[1] else "N")
name = sg.sgemm_f32_algo_name


def _operands(M, N, K, dist, seed, ta, tb, pad_a=0, pad_b=0):
    X = synthgen.matrix(M, K, seed=seed, stream=0, dist=dist)   # op(A)
    Y = synthgen.matrix(K, N, seed=seed, stream=1, dist=dist)   # op(B)
    C0 = synthgen.matrix(M, N, seed=seed, stream=2, dist=dist)
    As = stored(X, ta, (M if ta else K) + pad_a if pad_a else None)
    Bs = stored(Y, tb, (K if tb else N) + pad_b if pad_b else None)
    return As, Bs, C0


def _run(As, Bs, M, N, K, ta, tb, alpha, beta, C0, algo=sg.ALGO_AUTO, tile=None, **kw):
    log(f"[gpu] ex {'T' if ta else 'N'}{'T' if tb else 'N'} algo={name(algo)} tile={tile} "
        f"M={M} N={N} K={K} alpha={alpha} beta={beta} {kw}")
    d = Device(As, Bs, M, N, K, c_init=C0, **kw)
    d.run_ex(ta, tb, alpha, beta, algo=algo, tile=tile)
    C, guards = d.result()
    assert_guards(guards)
    return C


@pytest.mark.parametrize("layout", LAYOUTS, ids=lid)
@pytest.mark.parametrize("algo", TRANS_ALGOS, ids=name)
@pytest.mark.parametrize("shape", [(37, 29, 53), (130, 67, 129), (300, 517, 259), (20, 130, 90),
                                   (130, 20, 90), (6, 70, 45), (70, 6, 45)],
                         ids=lambda s: "x".join(map(str, s)))
def test_layouts_exact_integers(shape, algo, layout):
    M, N, K = shape
    ta, tb = layout
    As, Bs, C0 = _operands(M, N, K, "smallint", 500 + M + K, ta, tb)
    C = _run(As, Bs, M, N, K, ta, tb, 2.0, -1.0, C0, algo)
    check_ex(As, Bs, M, N, K, ta, tb, 2.0, -1.0, C0, C, f"{name(algo)} {lid(layout)}", exact=True)


@pytest.mark.parametrize("layout", LAYOUTS, ids=lid)
@pytest.mark.parametrize("algo", TRANS_ALGOS, ids=name)
def test_layouts_normal_padded_misaligned(algo, layout):
    M, N, K = 211, 333, 190
    ta, tb = layout
    As, Bs, C0 = _operands(M, N, K, "normal", 7, ta, tb, pad_a=5, pad_b=3)
    C = _run(As, Bs, M, N, K, ta, tb, -1.25, 0.375, C0, algo, ldc=N + 7, offset_elems=1)
    check_ex(As, Bs, M, N, K, ta, tb, -1.25, 0.375, C0, C, f"{name(algo)} {lid(layout)} padded")


@pytest.mark.parametrize("layout", LAYOUTS, ids=lid)
@pytest.mark.parametrize("tile", range(sg.sgemm_f32_mfma_tiles()), ids=sg.sgemm_f32_mfma_tile_name)
def test_tiles_all_layouts_exact(tile, layout):
    bm, bn, bk = (int(x) for x in sg.sgemm_f32_mfma_tile_name(tile).split()[0].split("x"))
    ta, tb = layout
    for (M, N, K) in [(2 * bm + 37, 2 * bn + 19, 9 * bk + 3), (bm + 1, 3, 6 * bk + 1)]:
        As, Bs, C0 = _operands(M, N, K, "smallint", 600 + tile, ta, tb)
        C = _run(As, Bs, M, N, K, ta, tb, 1.0, 0.0, C0, tile=tile)
        check_ex(As, Bs, M, N, K, ta, tb, 1.0, 0.0, C0, C, f"tile {tile} {lid(layout)}",
                 exact=True)
        C = _run(As, Bs, M, N, K, ta, tb, -2.0, 3.0, C0, tile=tile)
        check_ex(As, Bs, M, N, K, ta, tb, -2.0, 3.0, C0, C, f"tile {tile} {lid(layout)} ab",
                 exact=True)


@pytest.mark.parametrize("layout", LAYOUTS, ids=lid)
@pytest.mark.parametrize("tile", range(sg.sgemm_f32_mfma_tiles()), ids=sg.sgemm_f32_mfma_tile_name)
def test_tiles_long_k_exact(tile, layout):
    """Forty-one k windows (the last one partial) on a grid of nine blocks with
    ragged edges: one round of blocks over a long k, where the configurations that
    carry windows through a ring of register sets use it."""
    bm, bn, bk = (int(x) for x in sg.sgemm_f32_mfma_tile_name(tile).split()[0].split("x"))
    ta, tb = layout
    M, N, K = 2 * bm + 37, 2 * bn + 19, 40 * bk + 3
    As, Bs, C0 = _operands(M, N, K, "smallint", 650 + tile, ta, tb)
    C = _run(As, Bs, M, N, K, ta, tb, 2.0, -1.0, C0, tile=tile)
    check_ex(As, Bs, M, N, K, ta, tb, 2.0, -1.0, C0, C, f"tile {tile} {lid(layout)} long k",
             exact=True)


@pytest.mark.parametrize("layout", [(N_, N_), (T_, N_), (N_, T_)], ids=lid)
@pytest.mark.parametrize("windows", [(16, 0), (17, 0), (18, 0), (17, 5), (19, 1)],
                         ids=lambda w: f"w{w[0]}+{w[1]}")
@pytest.mark.parametrize("tile", [1, 3, 4, 5, 6, 7], ids=sg.sgemm_f32_mfma_tile_name)
def test_ring_window_counts_exact(tile, windows, layout):
    """Every configuration with a register ring, on four blocks (one round) at the
    smallest window counts that take the ring: 16, 17 and 18 whole windows leave
    each possible number of steady windows (0, 1 or 2) after the last whole group
    of two or three register sets, and a partial last window (k = 5 or 1 past the
    whole ones) adds a guarded window to the tail."""
    whole, extra = windows
    bm, bn, bk = (int(x) for x in sg.sgemm_f32_mfma_tile_name(tile).split()[0].split("x"))
    ta, tb = layout
    M, N, K = bm + 5, bn + 3, whole * bk + extra
    As, Bs, C0 = _operands(M, N, K, "smallint", 670 + tile + whole, ta, tb)
    C = _run(As, Bs, M, N, K, ta, tb, 1.0, -2.0, C0, tile=tile)
    check_ex(As, Bs, M, N, K, ta, tb, 1.0, -2.0, C0, C,
             f"tile {tile} {lid(layout)} {whole} windows + {extra}", exact=True)


@pytest.mark.parametrize("layout", [(N_, N_), (T_, T_)], ids=lid)
@pytest.mark.parametrize("tile", [4, 5], ids=sg.sgemm_f32_mfma_tile_name)
def test_tiles_many_rounds_long_k_sampled(tile, layout):
    """324 blocks (more than one per CU) over 101 k windows, the last one partial:
    the register ring is used on grids of several rounds when k is this long."""
    from gpu_helpers import sample_indices
    bm, bn, bk = (int(x) for x in sg.sgemm_f32_mfma_tile_name(tile).split()[0].split("x"))
    ta, tb = layout
    M, N, K = 17 * bm + 5, 17 * bn + 5, 100 * bk + 7
    As, Bs, C0 = _operands(M, N, K, "smallint", 660 + tile, ta, tb)
    C = _run(As, Bs, M, N, K, ta, tb, 1.0, 1.0, C0, tile=tile)
    r, c = sample_indices(M, N, rows=6, cols=6, elems=2048, seed=tile)
    check_ex(As, Bs, M, N, K, ta, tb, 1.0, 1.0, C0, C, f"tile {tile} {lid(layout)} rounds",
             exact=True, rows=r, cols=c)


@pytest.mark.parametrize("case", [(1, 3000, 1500, 39), (2, 777, 2049, 62), (1, 300, 4099, 31),
                                  (2, 5000, 257, 98)], ids=lambda c: "x".join(map(str, c)))
def test_few_rows_both_transposed_padded_a(case):
    """One or two rows of C with both operands transposed: the few-rows rung runs
    it as C^T = B^T op(A)^T on the few-columns kernel, with y = op(A)^T read from
    the stored A, whose rows (lda = M + pad) are far apart: y is gathered into
    LDS."""
    M, N, K, pad = case
    As, Bs, C0 = _operands(M, N, K, "smallint", 690 + K, T_, T_, pad_a=pad)
    for algo in (sg.ALGO_AUTO, sg.ALGO_SKINNY):
        C = _run(As, Bs, M, N, K, T_, T_, 3.0, -1.0, C0, algo)
        check_ex(As, Bs, M, N, K, T_, T_, 3.0, -1.0, C0, C, f"{name(algo)} TT {case}", exact=True)


@pytest.mark.parametrize("algo", NN_ONLY + TRANS_ALGOS, ids=name)
@pytest.mark.parametrize("shape", [(5, 300, 77), (300, 6, 77), (70, 90, 33)],
                         ids=lambda s: "x".join(map(str, s)))
def test_alpha_beta_untransposed(shape, algo):
    M, N, K = shape
    As, Bs, C0 = _operands(M, N, K, "normal", 40 + M, N_, N_)
    for alpha, beta in [(1.0, 1.0), (0.5, -2.0), (-3.0, 0.0)]:
        C = _run(As, Bs, M, N, K, N_, N_, alpha, beta, C0, algo)
        check_ex(As, Bs, M, N, K, N_, N_, alpha, beta, C0, C, f"{name(algo)} a={alpha} b={beta}")


@pytest.mark.parametrize("algo", NN_ONLY, ids=name)
def test_untransposed_only_rungs_reject_transposes(algo):
    M, N, K = 8, 8, 8
    As, Bs, C0 = _operands(M, N, K, "smallint", 1, T_, N_)
    d = Device(As, Bs, M, N, K, c_init=C0)
    with pytest.raises(sg.SgemmError):
        d.run_ex(T_, N_, 1.0, 0.0, algo=algo)
    C, guards = d.result()
    assert_guards(guards)
    assert np.array_equal(C, C0), "C changed by a rejected call"


@pytest.mark.parametrize("layout", LAYOUTS, ids=lid)
@pytest.mark.parametrize("algo", TRANS_ALGOS + NN_ONLY, ids=name)
def test_beta_zero_leaves_c_unread(algo, layout):
    """NaN in C must not reach the result when beta == 0."""
    ta, tb = layout
    if algo in NN_ONLY and layout != (N_, N_):
        pytest.skip("rung takes untransposed operands only")
    M, N, K = 67, 45, 31
    As, Bs, _ = _operands(M, N, K, "smallint", 3, ta, tb)
    nan_c = np.full((M, N), np.nan, dtype=np.float32)
    C = _run(As, Bs, M, N, K, ta, tb, 1.5, 0.0, nan_c, algo)
    assert np.all(np.isfinite(C))
    check_ex(As, Bs, M, N, K, ta, tb, 1.5, 0.0, None, C, f"{name(algo)} beta=0", exact=True)


@pytest.mark.parametrize("layout", LAYOUTS, ids=lid)
def test_product_free_cases(layout):
    """alpha == 0 or K == 0: C = beta*C and A, B are not read (NaN there stays out)."""
    ta, tb = layout
    M, N, K = 33, 21, 9
    As = np.full((K, M) if ta else (M, K), np.nan, dtype=np.float32)
    Bs = np.full((N, K) if tb else (K, N), np.nan, dtype=np.float32)
    C0 = synthgen.matrix(M, N, seed=9, stream=2, dist="smallint")
    C = _run(As, Bs, M, N, K, ta, tb, 0.0, 0.5, C0)
    assert np.array_equal(C, C0 * np.float32(0.5))
    C = _run(As, Bs, M, N, K, ta, tb, 0.0, 0.0, C0)
    assert np.all(C == 0)
    d = Device(As, Bs, M, N, 0, c_init=C0)
    d.run_ex(ta, tb, 1.0, -1.0)
    C, guards = d.result()
    assert_guards(guards)
    assert np.array_equal(C, -C0)


@pytest.mark.parametrize("algo", [sg.ALGO_AUTO, sg.ALGO_SKINNY], ids=name)
@pytest.mark.parametrize("shape", [(2, 4096, 4096), (2, 1000, 1023), (2, 37, 4093), (2, 515, 6)],
                         ids=lambda s: "x".join(map(str, s)))
def test_two_rows_both_transposed(shape, algo):
    """Two rows of C with both operands transposed and stored dense: the few-rows
    product runs as the few-columns kernel on C^T = B^T A^T, whose right operand
    (A as stored, K x 2 with lda = 2) has rows of two values; K % 4 != 0 leaves a
    tail of k rows after the whole vectors."""
    M, N, K = shape
    As, Bs, C0 = _operands(M, N, K, "smallint", 800 + N + K, T_, T_)
    assert As.shape == (K, 2) and Bs.shape == (N, K)
    for alpha, beta in [(1.0, 0.0), (2.0, -3.0)]:
        C = _run(As, Bs, M, N, K, T_, T_, alpha, beta, C0, algo)
        check_ex(As, Bs, M, N, K, T_, T_, alpha, beta, C0, C,
                 f"{name(algo)} TT {M}x{N}x{K} a={alpha} b={beta}", exact=True)


@pytest.mark.parametrize("layout", LAYOUTS, ids=lid)
def test_ragged_large_sampled(layout):
    """The ragged 4095 x 4097 x 1023 workload in every storage order, on sampled rows,
    columns and elements."""
    from gpu_helpers import sample_indices
    ta, tb = layout
    M, N, K = 4095, 4097, 1023
    As, Bs, C0 = _operands(M, N, K, "uniform_pm1", 4, ta, tb)
    C = _run(As, Bs, M, N, K, ta, tb, 1.0, 1.0, C0)
    r, c = sample_indices(M, N, rows=6, cols=6, elems=2048, seed=11)
    check_ex(As, Bs, M, N, K, ta, tb, 1.0, 1.0, C0, C, f"ragged {lid(layout)}", rows=r, cols=c)


@pytest.mark.parametrize("layout", [(N_, T_), (T_, N_), (T_, T_)], ids=lid)
@pytest.mark.parametrize("shape", [(2048, 3072, 4096), (8192, 8192, 8192)],
                         ids=lambda s: "x".join(map(str, s)))
def test_headline_workloads_transposed_sampled(shape, layout):
    """2048 x 3072 x 4096 and 8192^3 with transposed operands, as bench.py --layout
    times them: N(0,1) within the tolerance, and for the smaller one small integers
    bitwise, on sampled rows, columns and elements."""
    from gpu_helpers import sample_indices
    ta, tb = layout
    M, N, K = shape
    As, Bs, C0 = _operands(M, N, K, "normal", 3 if M == 2048 else 6, ta, tb)
    C = _run(As, Bs, M, N, K, ta, tb, 1.0, 0.0, C0)
    r, c = sample_indices(M, N, rows=4, cols=4, elems=2048, seed=13)
    check_ex(As, Bs, M, N, K, ta, tb, 1.0, 0.0, C0, C, f"{shape} {lid(layout)}", rows=r, cols=c)
    if M == 2048:
        As, Bs, C0 = _operands(M, N, K, "smallint", 33, ta, tb)
        C = _run(As, Bs, M, N, K, ta, tb, 2.0, -1.0, C0)
        check_ex(As, Bs, M, N, K, ta, tb, 2.0, -1.0, C0, C, f"{shape} {lid(layout)} int",
                 exact=True, rows=r, cols=c)


@pytest.mark.parametrize("layout", LAYOUTS, ids=lid)
def test_colmajor_entry(layout):
    """Column-major arrays, reference-BLAS argument order: the same product as the
    row-major general form of the transposes."""
    torch = pytest.importorskip("torch")
    ta, tb = layout
    M, N, K = 45, 38, 27
    X = synthgen.matrix(M, K, seed=12, stream=0, dist="smallint")
    Y = synthgen.matrix(K, N, seed=12, stream=1, dist="smallint")
    C0 = synthgen.matrix(M, N, seed=12, stream=2, dist="smallint")
    # column-major storage of op-operands: A_cm holds op(A) (or its transpose)
    A_cm = np.asfortranarray(X.T if ta else X)
    B_cm = np.asfortranarray(Y.T if tb else Y)
    lda, ldb, ldc = A_cm.shape[0], B_cm.shape[0], M
    dA = torch.from_numpy(A_cm.ravel(order="F").copy()).cuda()
    dB = torch.from_numpy(B_cm.ravel(order="F").copy()).cuda()
    dC = torch.from_numpy(np.asfortranarray(C0).ravel(order="F").copy()).cuda()
    st = sg.sgemm_f32_colmajor(ta, tb, M, N, K, 2.0, dA.data_ptr(), lda, dB.data_ptr(), ldb, -1.0,
                               dC.data_ptr(), ldc, torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    Cg = dC.cpu().numpy().reshape(N, M).T      # back from column-major
    exact = 2 * (X.astype(np.int64) @ Y.astype(np.int64)) - C0.astype(np.int64)
    assert np.array_equal(Cg.astype(np.int64), exact)


def test_torch_helper_transposed_views_and_scaling():
    torch = pytest.importorskip("torch")
    M, N, K = 77, 66, 55
    X = synthgen.matrix(M, K, seed=21, stream=0, dist="smallint")
    Y = synthgen.matrix(K, N, seed=21, stream=1, dist="smallint")
    C0 = synthgen.matrix(M, N, seed=21, stream=2, dist="smallint")
    exact = 3 * (X.astype(np.int64) @ Y.astype(np.int64)) - 2 * C0.astype(np.int64)
    Xt = torch.from_numpy(np.ascontiguousarray(X.T)).cuda()   # K x M storage
    Yt = torch.from_numpy(np.ascontiguousarray(Y.T)).cuda()   # N x K storage
    Xd = torch.from_numpy(X).cuda()
    Yd = torch.from_numpy(Y).cuda()
    for a, b in [(Xd, Yd), (Xt.t(), Yd), (Xd, Yt.t()), (Xt.t(), Yt.t())]:
        out = torch.from_numpy(C0.copy()).cuda()
        sg.matmul(a, b, out=out, alpha=3.0, beta=-2.0)
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy().astype(np.int64), exact)
    with pytest.raises(ValueError):
        sg.matmul(Xd, Yd, beta=1.0)


def _sweep_cases(n=48, seed=2024):
    """Seeded shapes for the automatic choice: sizes log-uniform over 1..1500 (every
    dimension below 9 a quarter of the time, so the few-row and few-column kernels
    and the edge strips come up), any storage order, padded row strides, and one of
    three alpha/beta pairs."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        dims = []
        for _ in range(3):
            if rng.random() < 0.25:
                dims.append(int(rng.integers(1, 9)))
            else:
                dims.append(int(np.exp(rng.uniform(np.log(9), np.log(1500)))))
        ta, tb = (int(x) for x in rng.integers(0, 2, 2))
        ab = [(1.0, 0.0), (2.0, -1.0), (0.5, 0.25)][int(rng.integers(0, 3))]
        pads = (int(rng.integers(0, 6)), int(rng.integers(0, 6)))
        cases.append((i, *dims, ta, tb, *ab, *pads))
    return cases


@pytest.mark.parametrize("case", _sweep_cases(), ids=lambda c: f"{c[0]}-{c[1]}x{c[2]}x{c[3]}")
def test_random_shapes_automatic_choice(case):
    """The automatic choice on seeded random shapes, bitwise on small integers (the
    alpha/beta pairs are exact in fp32 on integer data)."""
    _, M, N, K, ta, tb, alpha, beta, pad_a, pad_b = case
    As, Bs, C0 = _operands(M, N, K, "smallint", 700 + case[0], ta, tb, pad_a, pad_b)
    C = _run(As, Bs, M, N, K, ta, tb, alpha, beta, C0)
    check_ex(As, Bs, M, N, K, ta, tb, alpha, beta, C0, C,
             f"auto {lid((ta, tb))} {M}x{N}x{K}", exact=True)

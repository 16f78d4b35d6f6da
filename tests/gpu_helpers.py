"""Shared helpers of the GPU parity tests: seeded inputs, device upload through
torch (memory only), calls through the C ABI, and comparison with the oracle."""
from __future__ import annotations

import sys

import numpy as np

import dense_fp32_matrix_f32_amd as sg
import oracle
import synthgen

SENTINEL = np.float32(-7.25e30)   # guard value around C; never a product of test data


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a visible MI355X")
    return torch


def inputs(M, N, K, dist, seed, lda=None, ldb=None):
    """Host operands A (M x lda) and B (K x ldb); padding columns hold NaN."""
    if dist == "ones":
        A = synthgen.ones(M, K, ld=lda)
        B = synthgen.ones(K, N, ld=ldb)
    else:
        A = synthgen.matrix(M, K, seed=seed, stream=0, dist=dist, ld=lda)
        B = synthgen.matrix(K, N, seed=seed, stream=1, dist=dist, ld=ldb)
    return A, B


class Device:
    """Device copies of A, B and a C buffer with sentinel guard bands.

    C is allocated as (M + 2) x ldc with one sentinel row above and below the
    logical matrix; columns N..ldc-1 of every row also hold the sentinel.
    """

    def __init__(self, A, B, M, N, K, ldc=None, offset_elems=0, fill=SENTINEL, c_init=None):
        torch = torch_cuda()
        self.torch = torch
        self.M, self.N, self.K = M, N, K
        self.lda = A.shape[1]
        self.ldb = B.shape[1]
        self.ldc = max(ldc or N, 1)
        o = offset_elems
        self.a_buf = torch.from_numpy(np.concatenate([np.zeros(o, np.float32), A.ravel()])).cuda()
        self.b_buf = torch.from_numpy(np.concatenate([np.zeros(o, np.float32), B.ravel()])).cuda()
        self.c_buf = torch.full(((M + 2) * self.ldc + o,), float(fill), dtype=torch.float32,
                                device="cuda")
        self.a_ptr = self.a_buf.data_ptr() + 4 * o
        self.b_ptr = self.b_buf.data_ptr() + 4 * o
        self.c_ptr = self.c_buf.data_ptr() + 4 * (o + self.ldc)
        self.offset = o
        if c_init is not None:
            # the logical C (rows 1..M of the buffer, columns 0..N-1) starts as c_init
            view = self.c_buf[o + self.ldc:o + self.ldc + M * self.ldc].view(M, self.ldc)
            view[:, :N] = torch.from_numpy(np.ascontiguousarray(c_init, dtype=np.float32)).cuda()

    def run(self, algo=sg.ALGO_AUTO, stream=None):
        torch = self.torch
        s = stream if stream is not None else torch.cuda.current_stream()
        st = sg.sgemm_f32_algo(self.M, self.N, self.K, self.a_ptr, self.lda, self.b_ptr, self.ldb,
                               self.c_ptr, self.ldc, s.cuda_stream, algo)
        if st != 0:
            raise sg.SgemmError(st)
        s.synchronize()

    def run_tile(self, tile, stream=None):
        """The matrix-core rung with tile configuration `tile` forced."""
        torch = self.torch
        s = stream if stream is not None else torch.cuda.current_stream()
        st = sg.sgemm_f32_mfma_tile(self.M, self.N, self.K, self.a_ptr, self.lda, self.b_ptr,
                                    self.ldb, self.c_ptr, self.ldc, s.cuda_stream, tile)
        if st != 0:
            raise sg.SgemmError(st, "sgemm_f32_mfma_tile")
        s.synchronize()

    def run_ex(self, transa, transb, alpha, beta, algo=sg.ALGO_AUTO, tile=None, stream=None):
        """C = alpha*op(A)*op(B) + beta*C through sgemm_f32_ex_algo, or the matrix-core
        rung with configuration `tile`."""
        torch = self.torch
        s = stream if stream is not None else torch.cuda.current_stream()
        args = (transa, transb, self.M, self.N, self.K, alpha, self.a_ptr, self.lda, self.b_ptr,
                self.ldb, beta, self.c_ptr, self.ldc, s.cuda_stream)
        if tile is None:
            st = sg.sgemm_f32_ex_algo(*args, algo)
        else:
            st = sg.sgemm_f32_ex_mfma_tile(*args, tile)
        if st != 0:
            raise sg.SgemmError(st, "sgemm_f32_ex")
        s.synchronize()

    def result(self):
        """(C as M x N float32, guard-band contents) on the host."""
        full = self.c_buf.cpu().numpy()[self.offset:].reshape(self.M + 2, self.ldc)
        C = full[1:self.M + 1, :self.N].copy()
        guards = np.concatenate([full[0], full[self.M + 1], full[1:self.M + 1, self.N:].ravel()])
        return C, guards


def assert_guards(guards):
    bad = np.count_nonzero(guards.view(np.uint32) != SENTINEL.view(np.uint32))
    assert bad == 0, f"{bad} elements outside C were written"


def assert_close(Cg, Cref, S, what):
    ex = oracle.excess(Cg, Cref, S)
    worst = float(np.max(ex)) if ex.size else 0.0
    nbad = int(np.count_nonzero(ex > 1.0))
    assert nbad == 0, f"{what}: {nbad} elements beyond tolerance (worst excess {worst:.3g})"
    return worst


def sample_indices(M, N, rows=12, cols=12, elems=4096, seed=0):
    """Rows and columns to compare whole (edges, middles, random), plus random elements."""
    rng = np.random.default_rng(seed)
    rset = sorted(set([0, 1, M // 2, M - 2, M - 1] + list(rng.integers(0, M, rows))) &
                  set(range(M)))
    cset = sorted(set([0, 1, N // 2, N - 2, N - 1] + list(rng.integers(0, N, cols))) &
                  set(range(N)))
    r = [np.repeat(np.array(rset), N), np.tile(np.arange(M), len(cset)), rng.integers(0, M, elems)]
    c = [np.tile(np.arange(N), len(rset)), np.repeat(np.array(cset), M), rng.integers(0, N, elems)]
    return np.concatenate(r), np.concatenate(c)


def check_full(A, B, M, N, K, Cg, what, exact=False):
    Cref, S = oracle.sgemm(A[:, :K], B[:, :N])
    if exact:
        assert np.array_equal(Cg.astype(np.float64), Cref), f"{what}: not bitwise exact"
        return 0.0
    return assert_close(Cg, Cref, S, what)


def check_sampled(A, B, M, N, K, Cg, what, exact=False, seed=0):
    r, c = sample_indices(M, N, seed=seed)
    Cref, S = oracle.sgemm_elems(A[:, :K], B[:, :N], r, c)
    g = Cg[r, c]
    if exact:
        assert np.array_equal(g.astype(np.float64), Cref), f"{what}: sampled not bitwise exact"
        return 0.0
    return assert_close(g, Cref, S, what)


def stored(X, trans, ld=None):
    """The row-major array that holds X (rows x cols) as an operand passed with
    `trans`: X itself, or its transpose; padding columns hold NaN."""
    Y = np.ascontiguousarray(X.T) if trans else np.ascontiguousarray(X)
    if ld is None or ld == Y.shape[1]:
        return Y
    out = np.full((Y.shape[0], ld), np.nan, dtype=np.float32)
    out[:, :Y.shape[1]] = Y
    return out


def check_ex(As, Bs, M, N, K, ta, tb, alpha, beta, C0, Cg, what, exact=False, rows=None,
             cols=None):
    """Compare the GPU result of the general form with the oracle (whole, or the
    listed elements).  As and Bs are the stored arrays, possibly padded."""
    Av = As[:, :(M if ta else K)]
    Bv = Bs[:, :(K if tb else N)]
    Cref, S = oracle.sgemm_ex(Av, Bv, ta, tb, alpha, beta, C0, rows=rows, cols=cols)
    g = Cg if rows is None else Cg[rows, cols]
    if exact:
        assert np.array_equal(g.astype(np.float64), Cref), f"{what}: not bitwise exact"
        return 0.0
    return assert_close(g, Cref, S, what)

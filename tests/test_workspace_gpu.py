"""Split-k with a caller-provided workspace (sgemm_f32_ex_ws) against the oracle:
products with few blocks of C and a long k on the matrix cores, in every
storage order, with alpha and beta; bitwise on small-integer data.  Also: results reproducible run to run, the
workspace beyond the bytes the plan uses is never written, and a workspace that
is too small gives exactly the result of sgemm_f32_ex."""
import numpy as np
import pytest

import dense_fp32_matrix_f32_amd as sg
import oracle
import synthgen
from gpu_helpers import log, stored, torch_cuda

pytestmark = pytest.mark.gpu

N_, T_ = sg.OP_N, sg.OP_T
SENT = -7.25e30

# (M, N, K, layout): ragged edges, a partial last k window, every storage order
CASES = [(128, 128, 65536, (N_, N_)), (128, 128, 65536, (T_, T_)), (64, 64, 4096, (N_, T_)),
         (200, 150, 9000, (T_, N_)), (130, 67, 20001, (N_, N_)), (37, 300, 12000, (T_, T_))]
cid = lambda c: f"{c[0]}x{c[1]}x{c[2]}-{'T' if c[3][0] else 'N'}{'T' if c[3][1] else 'N'}"


def _setup(M, N, K, ta, tb, dist, seed):
    torch = torch_cuda()
    X = synthgen.matrix(M, K, seed=seed, stream=0, dist=dist)
    Y = synthgen.matrix(K, N, seed=seed, stream=1, dist=dist)
    C0 = synthgen.matrix(M, N, seed=seed, stream=2, dist="smallint")
    As, Bs = stored(X, ta), stored(Y, tb)
    return torch, As, Bs, C0, torch.from_numpy(As).cuda(), torch.from_numpy(Bs).cuda()


def _run_ws(torch, dA, dB, C0, M, N, K, ta, tb, alpha, beta, ws_floats):
    dC = torch.from_numpy(C0).cuda()
    ws = torch.full((max(ws_floats, 1),), SENT, dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream()
    st = sg.sgemm_f32_ex_ws(ta, tb, M, N, K, alpha, dA.data_ptr(), M if ta else K, dB.data_ptr(),
                            K if tb else N, beta, dC.data_ptr(), N, ws.data_ptr(), 4 * ws_floats,
                            s.cuda_stream)
    assert st == 0
    s.synchronize()
    return dC.cpu().numpy(), ws.cpu().numpy()


@pytest.mark.parametrize("case", CASES, ids=cid)
@pytest.mark.parametrize("dist", ["smallint", "normal"])
def test_split_k_matches_oracle(case, dist):
    M, N, K, (ta, tb) = case
    need = sg.sgemm_f32_workspace_size(ta, tb, M, N, K)
    assert need > 0 and need % (4 * M * N) == 0, "the plan no longer splits this shape"
    torch, As, Bs, C0, dA, dB = _setup(M, N, K, ta, tb, dist, 800 + M + N % 97)
    alpha, beta = (2.0, -1.0) if dist == "smallint" else (1.0, 0.0)
    log(f"[gpu] split-k {cid(case)} {dist} workspace {need} B")
    extra = 1000
    C, ws = _run_ws(torch, dA, dB, C0, M, N, K, ta, tb, alpha, beta, need // 4 + extra)
    assert np.all(ws[need // 4:] == np.float32(SENT)), "workspace written past the planned bytes"
    want, S = oracle.sgemm_ex(As, Bs, ta, tb, alpha, beta, C0)
    if dist == "smallint":
        assert np.array_equal(C.astype(np.float64), want)
    else:
        ex = oracle.excess(C, want, S)
        assert np.all(ex <= 1.0), f"{int(np.count_nonzero(ex > 1))} elements beyond tolerance"
    C2, _ = _run_ws(torch, dA, dB, C0, M, N, K, ta, tb, alpha, beta, need // 4)
    assert np.array_equal(C.view(np.uint32), C2.view(np.uint32)), "not reproducible"


@pytest.mark.parametrize("case", CASES[:1] + CASES[3:4], ids=cid)
def test_small_workspace_is_plain_ex(case):
    M, N, K, (ta, tb) = case
    need = sg.sgemm_f32_workspace_size(ta, tb, M, N, K)
    torch, As, Bs, C0, dA, dB = _setup(M, N, K, ta, tb, "normal", 5)
    C_small, ws = _run_ws(torch, dA, dB, C0, M, N, K, ta, tb, 1.0, 0.0, need // 4 - 1)
    assert np.all(ws == np.float32(SENT)), "a too small workspace was written"
    dC = torch.from_numpy(C0).cuda()
    s = torch.cuda.current_stream()
    assert sg.sgemm_f32_ex(ta, tb, M, N, K, 1.0, dA.data_ptr(), M if ta else K, dB.data_ptr(),
                           K if tb else N, 0.0, dC.data_ptr(), N, s.cuda_stream) == 0
    s.synchronize()
    assert np.array_equal(C_small.view(np.uint32), dC.cpu().numpy().view(np.uint32))


def test_matmul_helper_workspace():
    torch = torch_cuda()
    M, N, K = 128, 96, 30000
    A = synthgen.matrix(M, K, seed=44, stream=0, dist="smallint")
    B = synthgen.matrix(K, N, seed=44, stream=1, dist="smallint")
    At, Bt = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
    want, _ = oracle.sgemm(A, B)
    for ws in ("auto", torch.empty(sg.sgemm_f32_workspace_size(0, 0, M, N, K) // 4, device="cuda")):
        C = sg.matmul(At, Bt, workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(C.cpu().numpy().astype(np.float64), want)
    # on a side stream: the workspace and C that matmul allocates are released as
    # soon as it returns, while the product may still run there; new allocations
    # on the current stream, filled at once, must not land on them
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    for rep in range(3):
        C = sg.matmul(At, Bt, workspace="auto", stream=side)
        junk = [torch.full((1 << 20,), float("nan"), device="cuda") for _ in range(4)]
        side.synchronize()
        torch.cuda.synchronize()
        assert np.array_equal(C.cpu().numpy().astype(np.float64), want), rep
        del junk


def _reduce_groups(M, N, slices):
    """Plane groups per output element of the reduction for this plan: the fewest
    (up to 16, at most `slices`) that give 2048 work-groups of 256 work-items."""
    g = 1
    while g < 16 and 2 * g <= slices and (M * N * g + 255) // 256 < 2048:
        g *= 2
    return g


# one shape per plane grouping of the reduction (1, 2, 4, 8, 16 groups per element)
GROUP_CASES = [(1024, 512, 8192, 1), (512, 512, 32768, 2), (384, 384, 16384, 4),
               (256, 256, 16384, 8), (128, 128, 65536, 16)]


@pytest.mark.parametrize("case", GROUP_CASES, ids=lambda c: f"{c[0]}x{c[1]}x{c[2]}-g{c[3]}")
def test_reduction_groupings(case):
    """Every plane grouping of the reduction, on sampled outputs: whole rows and
    columns at both edges and a seeded scatter, with alpha and beta."""
    M, N, K, groups = case
    need = sg.sgemm_f32_workspace_size(N_, N_, M, N, K)
    assert need > 0 and need % (4 * M * N) == 0, "the plan no longer splits this shape"
    slices = need // (4 * M * N)
    assert _reduce_groups(M, N, slices) == groups, (slices, "the plan no longer gives this grouping")
    torch, As, Bs, C0, dA, dB = _setup(M, N, K, N_, N_, "normal", 900 + groups)
    log(f"[gpu] split-k reduction {M}x{N}x{K}, {slices} slices, {groups} groups")
    C, _ = _run_ws(torch, dA, dB, C0, M, N, K, N_, N_, 0.5, 2.0, need // 4)
    rng = np.random.default_rng(groups)
    rows = np.concatenate([np.repeat([0, M - 1], N), np.tile(np.arange(M), 2),
                           rng.integers(0, M, 4096)])
    cols = np.concatenate([np.tile(np.arange(N), 2), np.repeat([0, N - 1], M),
                           rng.integers(0, N, 4096)])
    want, S = oracle.sgemm_ex(As, Bs, False, False, 0.5, 2.0, C0, rows=rows, cols=cols)
    ex = oracle.excess(C[rows, cols], want, S)
    assert np.all(ex <= 1.0), f"{int(np.count_nonzero(ex > 1))} sampled elements beyond tolerance"


def _ws_sweep(n=12, seed=77):
    """Seeded shapes with few blocks of C and a long k: M, N in 1..300, K in 2000..30000,
    any storage order, one of three alpha/beta pairs."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        M, N = (int(x) for x in rng.integers(1, 301, 2))
        K = int(rng.integers(2000, 30001))
        ta, tb = (int(x) for x in rng.integers(0, 2, 2))
        ab = [(1.0, 0.0), (2.0, -1.0), (0.5, 0.25)][int(rng.integers(0, 3))]
        out.append((i, M, N, K, ta, tb, *ab))
    return out


@pytest.mark.parametrize("case", _ws_sweep(), ids=lambda c: f"{c[0]}-{c[1]}x{c[2]}x{c[3]}")
def test_random_shapes_with_workspace(case):
    """sgemm_f32_ex_ws with the workspace it asks for, split or not, bitwise on small
    integers; the workspace past the planned bytes stays untouched."""
    i, M, N, K, ta, tb, alpha, beta = case
    need = sg.sgemm_f32_workspace_size(ta, tb, M, N, K)
    torch, As, Bs, C0, dA, dB = _setup(M, N, K, ta, tb, "smallint", 1000 + i)
    log(f"[gpu] split-k sweep {M}x{N}x{K} {ta}{tb} alpha={alpha} beta={beta} workspace {need} B")
    C, ws = _run_ws(torch, dA, dB, C0, M, N, K, ta, tb, alpha, beta, need // 4 + 64)
    assert np.all(ws[need // 4:] == np.float32(SENT)), "workspace written past the planned bytes"
    want, _ = oracle.sgemm_ex(As, Bs, ta, tb, alpha, beta, C0)
    assert np.array_equal(C.astype(np.float64), want)

"""sgemm_f32_ex_noalloc (split-k planes in the library's own device array) against
sgemm_f32_ex_ws with a caller workspace, and both against the oracle: several calls
in a row on one GPU, each smaller than the one before, so every call runs on
scratch that still holds the previous call's planes."""
import numpy as np
import pytest

import dense_fp32_matrix_f32_amd as sg
from dense_fp32_matrix_f32_amd._binding import HIP_ERROR_INVALID_VALUE
import oracle
import synthgen
from gpu_helpers import log, sample_indices, stored, torch_cuda

pytestmark = pytest.mark.gpu

N_, T_ = sg.OP_N, sg.OP_T
SENT = np.float32(-7.25e30)
PAD = 5   # sentinel columns after each row of C


def _case(M, N, K, ta, tb, dist, seed):
    torch = torch_cuda()
    X = synthgen.matrix(M, K, seed=seed, stream=0, dist=dist)
    Y = synthgen.matrix(K, N, seed=seed, stream=1, dist=dist)
    C0 = synthgen.matrix(M, N, seed=seed, stream=2, dist="smallint")
    As, Bs = stored(X, ta), stored(Y, tb)
    return torch, As, Bs, C0, torch.from_numpy(As).cuda(), torch.from_numpy(Bs).cuda()


def _c_buffer(torch, C0):
    M, N = C0.shape
    full = np.full((M, N + PAD), SENT, dtype=np.float32)
    full[:, :N] = C0
    return torch.from_numpy(full).cuda()


def _call(entry, torch, dA, dB, C0, M, N, K, ta, tb, alpha, beta, ws=None):
    dC = _c_buffer(torch, C0)
    s = torch.cuda.current_stream()
    args = (ta, tb, M, N, K, alpha, dA.data_ptr(), M if ta else K, dB.data_ptr(),
            K if tb else N, beta, dC.data_ptr(), N + PAD)
    if entry == "noalloc":
        st = sg.sgemm_f32_ex_noalloc(*args, s.cuda_stream)
    elif entry == "ws":
        st = sg.sgemm_f32_ex_ws(*args, ws.data_ptr(), 4 * ws.numel(), s.cuda_stream)
    else:
        st = sg.sgemm_f32_ex(*args, s.cuda_stream)
    s.synchronize()
    full = dC.cpu().numpy()
    assert np.all(full[:, N:].view(np.uint32) == SENT.view(np.uint32)), f"{entry}: wrote past N"
    return st, full[:, :N].copy()


# Each call smaller than the one before; (M, N, K, layout, data, alpha, beta)
CALLS = [(512, 512, 32768, (N_, N_), "normal", 1.0, 0.0),
         (200, 150, 9000, (T_, N_), "smallint", 2.0, -1.0),
         (128, 64, 4096, (N_, T_), "smallint", 1.0, 1.0)]


def test_noalloc_matches_workspace_entry_on_successive_calls():
    torch = torch_cuda()
    for i, (M, N, K, (ta, tb), dist, alpha, beta) in enumerate(CALLS):
        need = sg.sgemm_f32_workspace_size(ta, tb, M, N, K)
        log(f"[gpu] noalloc call {i}: {M}x{N}x{K} {'T' if ta else 'N'}{'T' if tb else 'N'} "
            f"{dist} planes {need} B")
        assert 0 < need <= sg.SCRATCH_BYTES, "the planner no longer splits this shape"
        torch, As, Bs, C0, dA, dB = _case(M, N, K, ta, tb, dist, 900 + i)
        st, C_na = _call("noalloc", torch, dA, dB, C0, M, N, K, ta, tb, alpha, beta)
        assert st == 0, f"sgemm_f32_ex_noalloc returned {st}"
        ws = torch.full((need // 4,), float(SENT), dtype=torch.float32, device="cuda")
        st, C_ws = _call("ws", torch, dA, dB, C0, M, N, K, ta, tb, alpha, beta, ws=ws)
        assert st == 0
        assert np.array_equal(C_na.view(np.uint32), C_ws.view(np.uint32)), \
            f"call {i}: noalloc differs from the workspace entry point"
        if dist == "smallint":
            want, _ = oracle.sgemm_ex(As, Bs, ta, tb, alpha, beta, C0)
            assert np.array_equal(C_na.astype(np.float64), want), f"call {i}: not exact"
        else:
            r, c = sample_indices(M, N, rows=6, cols=6, elems=2048, seed=i)
            want, S = oracle.sgemm_ex(As, Bs, ta, tb, alpha, beta, C0, rows=r, cols=c)
            ex = oracle.excess(C_na[r, c], want, S)
            assert np.all(ex <= 1.0), f"call {i}: {int(np.count_nonzero(ex > 1))} beyond tolerance"


def test_noalloc_without_split_and_beyond_scratch():
    torch = torch_cuda()
    # no split planned: exactly sgemm_f32_ex
    M, N, K = 300, 200, 100
    assert sg.sgemm_f32_workspace_size(0, 0, M, N, K) == 0
    torch, As, Bs, C0, dA, dB = _case(M, N, K, N_, N_, "normal", 950)
    st, C_na = _call("noalloc", torch, dA, dB, C0, M, N, K, N_, N_, 1.5, 0.5)
    assert st == 0
    st, C_ex = _call("ex", torch, dA, dB, C0, M, N, K, N_, N_, 1.5, 0.5)
    assert st == 0 and np.array_equal(C_na.view(np.uint32), C_ex.view(np.uint32))
    # planes beyond the scratch array: refused, C untouched
    M, N, K = 768, 768, 65536
    assert sg.sgemm_f32_workspace_size(0, 0, M, N, K) > sg.SCRATCH_BYTES
    dA = torch.zeros((M, K), dtype=torch.float32, device="cuda")
    dB = torch.zeros((K, N), dtype=torch.float32, device="cuda")
    C0 = np.full((M, N), 3.0, dtype=np.float32)
    st, C = _call("noalloc", torch, dA, dB, C0, M, N, K, N_, N_, 1.0, 0.0)
    assert st == HIP_ERROR_INVALID_VALUE, f"expected hipErrorInvalidValue, got {st}"
    assert np.all(C == 3.0)


def test_noalloc_captured_in_a_graph():
    """Calls recorded under HIP graph capture (the callers the entry point is for):
    two split products whose planes share the static array, and one without a
    split, all accumulating into C.  The graph is replayed three times; between
    replays an eager split call of another shape overwrites the array and the
    operands change.  Every replay is checked bitwise against the oracle on small
    integers."""
    torch = torch_cuda()
    shapes = [(128, 96, 20000, N_, N_), (200, 150, 9000, T_, N_), (300, 200, 100, N_, T_)]
    cases = []
    for i, (M, N, K, ta, tb) in enumerate(shapes):
        torch, As, Bs, C0, dA, dB = _case(M, N, K, ta, tb, "smallint", 970 + i)
        dC = torch.from_numpy(C0.copy()).cuda()
        cases.append(dict(M=M, N=N, K=K, ta=ta, tb=tb, As=As, Bs=Bs, C0=C0, dA=dA, dB=dB, dC=dC))
    assert sg.sgemm_f32_workspace_size(N_, N_, 128, 96, 20000) > 0
    assert sg.sgemm_f32_workspace_size(T_, N_, 200, 150, 9000) > 0
    assert sg.sgemm_f32_workspace_size(N_, T_, 300, 200, 100) == 0
    # another split shape, run eagerly between replays (the array's address on
    # this device is looked up by the first call, made here before the capture)
    eA = torch.from_numpy(synthgen.matrix(512, 32768, seed=980, stream=0, dist="smallint")).cuda()
    eB = torch.from_numpy(synthgen.matrix(32768, 512, seed=980, stream=1, dist="smallint")).cuda()
    eC = torch.empty((512, 512), dtype=torch.float32, device="cuda")

    def eager_split():
        st = sg.sgemm_f32_ex_noalloc(N_, N_, 512, 512, 32768, 1.0, eA.data_ptr(), 32768,
                                     eB.data_ptr(), 512, 0.0, eC.data_ptr(), 512,
                                     torch.cuda.current_stream().cuda_stream)
        assert st == 0

    def call(c, s):
        M, N, K, ta, tb = c["M"], c["N"], c["K"], c["ta"], c["tb"]
        return sg.sgemm_f32_ex_noalloc(ta, tb, M, N, K, 1.0, c["dA"].data_ptr(),
                                       M if ta else K, c["dB"].data_ptr(), K if tb else N,
                                       1.0, c["dC"].data_ptr(), N, s)

    eager_split()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        s = torch.cuda.current_stream().cuda_stream
        for c in cases:
            assert call(c, s) == 0
    for replay in range(3):
        log(f"[gpu] noalloc graph replay {replay}")
        graph.replay()
        torch.cuda.synchronize()
        for c in cases:
            got = c["dC"].cpu().numpy()
            want, _ = oracle.sgemm_ex(c["As"], c["Bs"], c["ta"], c["tb"], 1.0, 1.0, c["C0"])
            assert np.array_equal(got.astype(np.float64), want), \
                (c["M"], c["N"], c["K"], replay)
            c["C0"] = got
            # eager work between replays: new operands for the next replay
            c["dA"].mul_(-1.0)
            c["As"] = c["dA"].cpu().numpy()
        eager_split()
        torch.cuda.synchronize()
    r, c = sample_indices(512, 512, rows=4, cols=4, elems=2048, seed=7)
    want, _ = oracle.sgemm_ex(eA.cpu().numpy(), eB.cpu().numpy(), 0, 0, 1.0, 0.0,
                              np.zeros((512, 512), np.float32), rows=r, cols=c)
    assert np.array_equal(eC.cpu().numpy()[r, c].astype(np.float64), want)

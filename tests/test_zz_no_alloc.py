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

"""The C ABI under HIP graph capture and on concurrent streams.

The library allocates nothing and never synchronizes, so a sequence of calls can
be captured into a graph and replayed.  The captured sequence covers every
kernel family the automatic choice launches: blocks of the matrix cores, a
product split into blocks and an edge strip (two launches), the few-rows and
few-columns streaming kernels, C = beta*C for K = 0, accumulation into C
(beta = 1), and split-k through a workspace.  The graph is replayed several times with eager work and
synchronizations in between (the operands change between replays); every replay
is compared with the oracle, bitwise on small-integer data.  A second test runs
products on two streams at once, a third from four host threads at once.
"""
import numpy as np
import pytest

import dense_fp32_matrix_f32_amd as sg
import oracle
import synthgen
from gpu_helpers import log, sample_indices, torch_cuda

pytestmark = pytest.mark.gpu

# (M, N, K, beta); the last one runs split-k through a workspace
CAPTURED = [(1000, 1100, 700, 0.0), (2049, 4097, 1023, 0.0), (1, 2049, 515, 0.0),
            (3000, 3, 700, 0.0), (100, 100, 0, 0.0), (300, 200, 150, 1.0), (128, 96, 20000, 1.0)]


def _exact(A, B, beta, C0, rows=None, cols=None):
    C, _ = oracle.sgemm_ex(A, B, 0, 0, 1.0, beta, C0, rows=rows, cols=cols)
    return C


def _elements(M, N, seed):
    if M * N <= 2_000_000:
        return None, None
    r, c = sample_indices(M, N, rows=4, cols=4, elems=2048, seed=seed)
    # the edge strip of a split product: its last columns and rows
    r = np.concatenate([r, np.repeat(np.arange(M), 2), np.repeat(np.arange(M - 2, M), N)])
    c = np.concatenate([c, np.tile(np.arange(N - 2, N), M), np.tile(np.arange(N), 2)])
    return r, c


def test_graph_capture_and_replay():
    torch = torch_cuda()
    cases = []
    for i, (M, N, K, beta) in enumerate(CAPTURED):
        if K > 0:
            A = synthgen.matrix(M, K, seed=90 + i, stream=0, dist="smallint")
            B = synthgen.matrix(K, N, seed=90 + i, stream=1, dist="smallint")
        else:
            A, B = np.zeros((M, 0), np.float32), np.zeros((0, N), np.float32)
        C0 = synthgen.matrix(M, N, seed=90 + i, stream=2, dist="smallint")
        dA = torch.from_numpy(A).cuda() if A.size else torch.zeros(1, device="cuda")
        dB = torch.from_numpy(B).cuda() if B.size else torch.zeros(1, device="cuda")
        dC = torch.from_numpy(C0).cuda()
        cases.append(dict(M=M, N=N, K=K, beta=beta, A=A, B=B, C0=C0, dA=dA, dB=dB, dC=dC))
    torch.cuda.synchronize()

    last = cases[-1]
    need = sg.sgemm_f32_workspace_size(0, 0, last["M"], last["N"], last["K"])
    assert need > 0
    ws = torch.empty(need // 4, dtype=torch.float32, device="cuda")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        s = torch.cuda.current_stream().cuda_stream
        for c in cases[:-1]:
            st = sg.sgemm_f32_ex(0, 0, c["M"], c["N"], c["K"], 1.0, c["dA"].data_ptr(),
                                 max(c["K"], 1), c["dB"].data_ptr(), c["N"], c["beta"],
                                 c["dC"].data_ptr(), c["N"], s)
            assert st == 0
        st = sg.sgemm_f32_ex_ws(0, 0, last["M"], last["N"], last["K"], 1.0, last["dA"].data_ptr(),
                                last["K"], last["dB"].data_ptr(), last["N"], last["beta"],
                                last["dC"].data_ptr(), last["N"], ws.data_ptr(), need, s)
        assert st == 0
    # capture records the launches without running them
    for replay in range(3):
        log(f"[gpu] graph replay {replay}")
        graph.replay()
        torch.cuda.synchronize()
        for c in cases:
            M, N = c["M"], c["N"]
            got = c["dC"].cpu().numpy()
            rows, cols = _elements(M, N, replay)
            want = _exact(c["A"], c["B"], c["beta"], c["C0"], rows, cols)
            g = got if rows is None else got[rows, cols]
            assert np.array_equal(g.astype(np.float64), want), (M, N, c["K"], replay)
            c["C0"] = got  # beta = 1 accumulates from here
        # eager work between replays: new operands for the next replay
        for c in cases:
            if c["K"] > 0:
                c["dA"].mul_(-1.0)
                c["A"] = c["dA"].cpu().numpy()
        torch.cuda.synchronize()


def test_concurrent_streams():
    torch = torch_cuda()
    shapes = [(700, 900, 650), (1, 4096, 1500), (2049, 4097, 300), (1500, 5, 900)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    work = []
    for i, (M, N, K) in enumerate(shapes):
        A = synthgen.matrix(M, K, seed=120 + i, stream=0, dist="smallint")
        B = synthgen.matrix(K, N, seed=120 + i, stream=1, dist="smallint")
        dA, dB = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
        outs = [torch.full((M, N), float("nan"), device="cuda") for _ in streams]
        work.append((M, N, K, A, B, dA, dB, outs))
    torch.cuda.synchronize()
    log("[gpu] concurrent streams")
    for rep in range(4):
        for M, N, K, A, B, dA, dB, outs in work:
            for st, out in zip(streams, outs):
                assert sg.sgemm_f32(M, N, K, dA.data_ptr(), K, dB.data_ptr(), N, out.data_ptr(),
                                    N, st.cuda_stream) == 0
    torch.cuda.synchronize()
    for M, N, K, A, B, dA, dB, outs in work:
        rows, cols = _elements(M, N, 0)
        want = _exact(A, B, 0.0, None, rows, cols)
        for out in outs:
            got = out.cpu().numpy()
            g = got if rows is None else got[rows, cols]
            assert np.array_equal(g.astype(np.float64), want), (M, N, K)


def test_host_threads():
    """Four host threads call the library at once, each on its own stream with its
    own outputs and workspace: blocks of the matrix cores, the few-rows kernel, a
    product with an edge strip, and split-k through a workspace."""
    import threading

    torch = torch_cuda()
    shapes = [(700, 900, 650), (1, 4096, 1500), (2049, 4097, 300), (128, 96, 20000)]
    inputs = []
    for i, (M, N, K) in enumerate(shapes):
        A = synthgen.matrix(M, K, seed=140 + i, stream=0, dist="smallint")
        B = synthgen.matrix(K, N, seed=140 + i, stream=1, dist="smallint")
        inputs.append((M, N, K, A, B, torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()))
    threads_n = 4
    streams = [torch.cuda.Stream() for _ in range(threads_n)]
    outs = [[torch.full((M, N), float("nan"), device="cuda") for (M, N, K, *_) in inputs]
            for _ in range(threads_n)]
    ws_bytes = [sg.sgemm_f32_workspace_size(0, 0, M, N, K) for (M, N, K, *_) in inputs]
    assert ws_bytes[-1] > 0, "the last shape should split k"
    wss = [torch.empty(max(ws_bytes) // 4 + 1, device="cuda") for _ in range(threads_n)]
    torch.cuda.synchronize()
    errors = []

    def worker(t):
        try:
            for rep in range(10):
                for j, (M, N, K, A, B, dA, dB) in enumerate(inputs):
                    st = sg.sgemm_f32_ex_ws(0, 0, M, N, K, 1.0, dA.data_ptr(), K, dB.data_ptr(), N,
                                            0.0, outs[t][j].data_ptr(), N, wss[t].data_ptr(),
                                            ws_bytes[j], streams[t].cuda_stream)
                    if st != 0:
                        errors.append((t, j, st))
        except Exception as e:  # reported below, on the main thread
            errors.append((t, repr(e)))

    log(f"[gpu] {threads_n} host threads")
    pool = [threading.Thread(target=worker, args=(t,)) for t in range(threads_n)]
    for th in pool:
        th.start()
    for th in pool:
        th.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for j, (M, N, K, A, B, dA, dB) in enumerate(inputs):
        rows, cols = _elements(M, N, j)
        want = _exact(A, B, 0.0, None, rows, cols)
        for t in range(threads_n):
            got = outs[t][j].cpu().numpy()
            g = got if rows is None else got[rows, cols]
            assert np.array_equal(g.astype(np.float64), want), (t, M, N, K)

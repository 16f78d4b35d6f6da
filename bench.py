"""Benchmark of the fp32 matrix product on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--shape M,N,K] [--algo NAME]

One step is one call of sgemm_f32 (the whole product) on inputs already resident
in HBM.  The default workload is C = A·B with M = N = K = 8192 and N(0,1) inputs
(the compute-bound point); the 2048 x 3072 x 4096 product (A 2048 x 4096, B 4096 x
3072) is timed after it and reported under "also".  Rank 0 prints one JSON line.

Throughput is 2MNK / t (page "CUDA算子优化(4)：矩阵乘法", section "计算强度": 2K flops
per output element); the algorithmic byte count is 4(MK + KN + MN) (same section),
used for the intensity I = MNK / (2(MK + KN + MN)).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_FP32_TFLOPS = 157.3      # MI355X dense fp32 (matrix and vector), 2.4 GHz
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 matrix cores
SPLIT_PART_PRODUCTS = 6       # bf16 part products per fp32 product on the split-precision rung
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "sgemm_mfma_8192_traffic.txt")
KERNEL_SOURCES = ["dense_fp32_matrix_f32_amd/csrc/mfma_kernel.h",
                  "dense_fp32_matrix_f32_amd/csrc/mfma_nn.hip",
                  "dense_fp32_matrix_f32_amd/csrc/mfma.hip",
                  "dense_fp32_matrix_f32_amd/csrc/tile_order.h",
                  "dense_fp32_matrix_f32_amd/csrc/internal.h"]


def algorithmic_flops(M: int, N: int, K: int) -> int:
    """2MNK: K multiplies and K adds per output element."""
    return 2 * M * N * K


def algorithmic_bytes(M: int, N: int, K: int) -> int:
    """4(MK + KN + MN): read A and B once, write C once, in fp32."""
    return 4 * (M * K + K * N + M * N)


def intensity(M: int, N: int, K: int) -> float:
    """Flops per byte, MNK / (2(MK + KN + MN)); N/6 for a square product."""
    return algorithmic_flops(M, N, K) / algorithmic_bytes(M, N, K)


def naive_global_reads(n: int) -> int:
    """Element reads of the one-thread-per-output kernel on an n x n product: 2n^3."""
    return 2 * n ** 3


def tiled_global_reads(n: int, tile: int) -> int:
    """Element reads of the tiled kernel: every loaded element serves `tile` outputs."""
    return 2 * n ** 3 // tile


def tile_intensity(tm: int, tn: int) -> float:
    """Flops per byte of one tm x tn tile step (page "CUDA算子优化(4)：矩阵乘法",
    section "版本V1共享内存分块"): 2*tm*tn*tk / ((tm*tk + tn*tk)*4)."""
    return 2 * tm * tn / ((tm + tn) * 4)


def code_tokens(text: str) -> str:
    """C++ source without comments and with whitespace runs collapsed, so that a
    change to comments or layout alone leaves the hash below unchanged (string
    literals in these files hold no comment markers)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash() -> str:
    """Hash of the code of the kernel sources (comments and whitespace ignored)."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            h.update(code_tokens(f.read()).encode())
    return h.hexdigest()[:16]


def read_traffic():
    """Bytes per launch between the L2 caches and the data fabric, from rocprofv3
    FETCH_SIZE and WRITE_SIZE scaled by a copy-kernel calibration, if they were
    taken on the current kernel source; else None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    with open(TRAFFIC_FILE, encoding="utf-8") as f:
        for line in f:
            if "=" in line and not line.lstrip().startswith("#"):
                k, v = line.split("=", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    try:
        return int(float(vals["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def split_record(flops: int, ms: float) -> dict:
    """Throughput of the split-precision rung: the fp32 product's 2MNK flops per second,
    and the bf16 matrix-core work it issues (six part products, 6 * 2MNK flops) as a
    fraction of the bf16 matrix peak, the roofline of the units it runs on."""
    fp32_eq = flops / (ms * 1e-3) / 1e12
    bf16 = SPLIT_PART_PRODUCTS * fp32_eq
    return {"kernel_ms": round(ms, 5), "fp32_equivalent_tflops": round(fp32_eq, 3),
            "bf16_mfma_tflops": round(bf16, 2), "peak_bf16_tflops": PEAK_BF16_TFLOPS,
            "pct_bf16_peak": round(100 * bf16 / PEAK_BF16_TFLOPS, 2)}


def host_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def make_inputs(torch, M, N, K, seed, dist="normal", layout=(0, 0)):
    """Seeded host operands and their device copies.  With a transposed layout the
    stored arrays are K x M (A) and N x K (B)."""
    import synthgen
    ta, tb = layout
    A = synthgen.matrix(K if ta else M, M if ta else K, seed=seed, stream=0, dist=dist)
    B = synthgen.matrix(N if tb else K, K if tb else N, seed=seed, stream=1, dist=dist)
    dA = torch.from_numpy(A).cuda()
    dB = torch.from_numpy(B).cuda()
    dC = torch.empty((M, N), dtype=torch.float32, device="cuda")
    return A, B, dA, dB, dC


def time_product(torch, sg, M, N, K, dA, dB, dC, algo, steps, warmup, layout=(0, 0),
                 workspace=None, sclk_log=None):
    """Warm-up, then `steps` timed launches back to back.  Returns the wall clock
    between two full synchronisations (seconds) and the average kernel time (ms):
    one HIP event pair on the launch stream around all timed launches, divided by
    their number.  No event sits between two launches: an event pair per launch
    opens a gap of about 10 us between kernels, half of which it would count as
    kernel time, while back-to-back launches run with no gap.  dB may be a list of
    device tensors, used in turn (B rotated over several buffers).  With a
    workspace tensor, the product goes through sgemm_f32_ex_ws.  With a list as
    sclk_log, the clock readings sampled while the timed launches run are appended."""
    stream = torch.cuda.current_stream()
    ta, tb = layout
    lda, ldb, ldc = (M if ta else K), (K if tb else N), N
    bufs = dB if isinstance(dB, (list, tuple)) else [dB]
    turn = [0]

    def call():
        b = bufs[turn[0] % len(bufs)].data_ptr()
        turn[0] += 1
        if workspace is not None:
            st = sg.sgemm_f32_ex_ws(ta, tb, M, N, K, 1.0, dA.data_ptr(), lda, b, ldb,
                                    0.0, dC.data_ptr(), ldc, workspace.data_ptr(),
                                    4 * workspace.numel(), stream.cuda_stream)
        elif layout == (0, 0):
            st = sg.sgemm_f32_algo(M, N, K, dA.data_ptr(), lda, b, ldb,
                                   dC.data_ptr(), ldc, stream.cuda_stream, algo)
        else:
            st = sg.sgemm_f32_ex_algo(ta, tb, M, N, K, 1.0, dA.data_ptr(), lda, b,
                                      ldb, 0.0, dC.data_ptr(), ldc, stream.cuda_stream, algo)
        if st != 0:
            raise sg.SgemmError(st)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    sampler = ClockSampler(torch) if sclk_log is not None else None
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        call()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if sampler is not None:
        sclk_log.append(sampler.stop())
    return wall, start.elapsed_time(end) / steps


def cpu_baseline(A, B, M, N, K, budget_s: float):
    """Time the oracle on whole rows of C until about `budget_s` of CPU time is spent."""
    import numpy as np

    import oracle
    threads = host_threads()
    row_cost = N * K
    # calibrate with one row per thread
    rows = threads
    r = np.repeat(np.arange(rows) * (M // max(rows, 1)), N)
    c = np.tile(np.arange(N), rows)
    t0 = time.perf_counter()
    oracle.sgemm_elems(A[:, :K], B[:, :N], r, c, threads=threads)
    t1 = time.perf_counter() - t0
    per_row = t1 / rows
    more = max(0, int((budget_s - t1) / max(per_row, 1e-9)))
    more = min(more, M - rows)
    if more > 0:
        r2 = np.repeat(np.linspace(0, M - 1, more).astype(np.int64), N)
        c2 = np.tile(np.arange(N), more)
        t0 = time.perf_counter()
        oracle.sgemm_elems(A[:, :K], B[:, :N], r2, c2, threads=threads)
        t2 = time.perf_counter() - t0
        rows_total, secs = rows + more, t1 + t2
    else:
        rows_total, secs = rows, t1
    flops = 2.0 * rows_total * row_cost
    return {"value": flops / secs / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{rows_total} whole rows of C ({rows_total}x{N} outputs, {K}-term fp64 sums) "
                      f"of the {M}x{N}x{K} product in {secs:.1f} s"}


def cpu_blocked(A, B, M, N, K, reps: int = 1):
    """Time the blocked multi-threaded host SGEMM on the whole product (best of reps)."""
    import hostsgemm
    threads = hostsgemm.threads_available()
    best = None
    for _ in range(reps):
        t0 = time.perf_counter()
        hostsgemm.sgemm(A[:, :K], B[:, :N], threads=threads)
        dt = time.perf_counter() - t0
        best = dt if best is None else min(best, dt)
    return {"value": algorithmic_flops(M, N, K) / best / 1e12, "unit": "TFLOP/s",
            "cores": threads, "kind": "blocked fp32 host SGEMM (packed panels, 6x16 "
            "micro-kernel, row ranges per thread)", "sample": f"whole {M}x{N}x{K} product, "
            f"{best * 1e3:.1f} ms"}


def ladder(torch, sg, M, N, K, args):
    """Kernel time of each algorithm on one product (warm-up by time, as above)."""
    _, _, dA, dB, dC = make_inputs(torch, M, N, K, args.seed)
    flops = algorithmic_flops(M, N, K)
    nbytes = algorithmic_bytes(M, N, K)
    for name, algo in sg.ALGOS.items():
        if algo == sg.ALGO_AUTO:
            continue
        # one probe launch sizes the warm-up and the timed count
        _, probe = time_product(torch, sg, M, N, K, dA, dB, dC, algo, 1, 1)
        est = max(probe, 1e-3)
        warm = max(args.warmup, min(2000, int(300 / est)))
        steps = max(args.steps, min(2000, int(200 / est)))
        _, avg = time_product(torch, sg, M, N, K, dA, dB, dC, algo, steps, warm)
        print(json.dumps({"shape": [M, N, K], "algo": name, "kernel_ms_avg": round(avg, 5),
                          "tflops": round(flops / (avg * 1e-3) / 1e12, 3),
                          "pct_fp32_peak": round(100 * flops / (avg * 1e-3) / 1e12 /
                                                 PEAK_FP32_TFLOPS, 2),
                          "gbs": round(nbytes / (avg * 1e-3) / 1e9, 1),
                          "pct_hbm_peak": round(100 * nbytes / (avg * 1e-3) / 1e9 / PEAK_HBM_GBS,
                                                2),
                          "steps": steps, "warmup": warm}), flush=True)


# The five workloads: name, M, N, K, input distribution, seed (A is stream 0 and
# B stream 1 of the seeded generator).
CONFIGS = [("c1", 512, 512, 512, "normal", 1), ("c2", 1024, 1024, 1024, "normal", 2),
           ("c3", 2048, 3072, 4096, "normal", 3), ("c4a", 4095, 4097, 1023, "uniform_pm1", 4),
           ("c4b", 1, 4096, 4096, "uniform_pm1", 5), ("c5", 8192, 8192, 8192, "normal", 6)]


def _check(status, sg):
    if status != 0:
        raise sg.SgemmError(status)


def _sclk_path(torch):
    p = torch.cuda.get_device_properties(0)
    return (f"/sys/bus/pci/devices/{p.pci_domain_id:04x}:{p.pci_bus_id:02x}:"
            f"{p.pci_device_id:02x}.0/pp_dpm_sclk")


def gpu_sclk(torch):
    """The shader clock that the driver marks as current for device 0 (MHz), or None.
    On MI355X this is the power controller's running average, which lags the clock
    the kernels run at by about a second; the clock during a kernel comes from the
    counters (GRBM_GUI_ACTIVE over the kernel time)."""
    try:
        with open(_sclk_path(torch)) as f:
            for line in f:
                if line.rstrip().endswith("*"):
                    return int(line.split(":", 1)[1].strip(" *\n").lower().replace("mhz", ""))
    except Exception:  # noqa: BLE001 -- informational only
        return None
    return None


class ClockSampler:
    """Reads gpu_sclk every 2 ms on a host thread until stop(); returns the samples'
    count, maximum and last value."""

    def __init__(self, torch):
        import threading
        self.torch, self.samples, self.done = torch, [], False
        self.thread = threading.Thread(target=self._run, daemon=True)
        self.thread.start()

    def _run(self):
        while not self.done:
            v = gpu_sclk(self.torch)
            if v is not None:
                self.samples.append(v)
            time.sleep(0.002)

    def stop(self):
        self.done = True
        self.thread.join()
        s = self.samples
        return {"samples": len(s), "max_mhz": max(s) if s else None,
                "last_mhz": s[-1] if s else None}


def timed_launches(torch, stream, launch, warm_ms=300.0, timed_ms=200.0, min_steps=20,
                   regions=5):
    """Average kernel time (ms) of back-to-back launches, one value per region: a
    time-based warm-up, then `regions` runs of launches, each timed by one HIP event
    pair on the stream around the whole run (no event between two launches)."""
    def run(n):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(n):
            launch()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n
    est = max(run(3), 1e-3)
    run(max(1, min(20000, int(warm_ms / est))))
    n = max(min_steps, min(20000, int(timed_ms / est / regions)))
    return [run(n) for _ in range(regions)], n * regions


def launch_floor(torch, sg):
    """Back-to-back time of the smallest launches: the fixed cost a product pays
    whatever its size (under rocprofv3 --kernel-trace the kernels' own durations
    come with it).  The tile ids are those of sgemm_f32_mfma_tile_name()."""
    import statistics

    stream = torch.cuda.current_stream()
    n = 1 << 20
    A = torch.randn(n, device="cuda")
    B = torch.randn(n, device="cuda")
    C = torch.empty(n, device="cuda")
    t512 = sg.sgemm_f32_mfma_select(512, 512, 512)
    t1024 = sg.sgemm_f32_mfma_select(1024, 1024, 1024)
    bk512 = int(sg.sgemm_f32_mfma_tile_name(t512).split()[0].split("x")[2])
    bk1024 = int(sg.sgemm_f32_mfma_tile_name(t1024).split()[0].split("x")[2])
    cases = [("C = 0 (512 x 512, K = 0)", (512, 512, 0, None)), ("1 x 1 x 1", (1, 1, 1, None))]
    for t, bk, m in ((t512, bk512, 512), (t1024, bk1024, 1024)):
        bm = int(sg.sgemm_f32_mfma_tile_name(t).split("x")[0])
        cases.append((f"tile {t}: one block, one window", (bm, bm, bk, t)))
        cases.append((f"tile {t}: {m} x {m} x {bk}, one window per block", (m, m, bk, t)))
        cases.append((f"tile {t}: {m} x {m} x {2 * bk}, two windows per block", (m, m, 2 * bk, t)))
    for name, (M, N, K, tile) in cases:
        lda = max(K, 1)
        C[:1].zero_()  # a torch kernel between the cases marks their boundaries in a kernel trace

        def launch():
            if tile is None:
                st = sg.sgemm_f32(M, N, K, A.data_ptr(), lda, B.data_ptr(), N, C.data_ptr(), N,
                                  stream.cuda_stream)
            else:
                st = sg.sgemm_f32_mfma_tile(M, N, K, A.data_ptr(), lda, B.data_ptr(), N,
                                            C.data_ptr(), N, stream.cuda_stream, tile)
            if st != 0:
                raise sg.SgemmError(st)

        kms, launches = timed_launches(torch, stream, launch, warm_ms=50.0, timed_ms=50.0)
        print(json.dumps({"launch": name, "shape": [M, N, K], "tile": tile,
                          "us_median": round(statistics.median(kms) * 1e3, 3),
                          "launches": launches,
                          "timing": "one HIP event pair around each of 5 runs of back-to-back "
                                    "launches"}), flush=True)


def config_report(torch, sg, args):
    """One JSON line per workload: kernel time (median, mean, min of per-launch
    events), TFLOP/s and GB/s against the peaks, the algorithm and tile used; for
    the 1 x 4096 x 4096 product also with B rotated over five buffers (320 MB, more
    than the 256 MB Infinity Cache), and for 512^3 and 1024^3 the oracle on one
    host thread and on all of them."""
    import statistics

    stream = torch.cuda.current_stream()
    print(json.dumps({"sclk_before": gpu_sclk(torch)}), flush=True)
    for name, M, N, K, dist, seed in CONFIGS:
        A, B, dA, dB, dC = make_inputs(torch, M, N, K, seed, dist)
        algo = sg.sgemm_f32_select(M, N, K, dA.data_ptr(), K, dB.data_ptr(), N, dC.data_ptr(), N)

        def launch(b_ptr=None):
            st = sg.sgemm_f32(M, N, K, dA.data_ptr(), K, b_ptr or dB.data_ptr(), N,
                              dC.data_ptr(), N, stream.cuda_stream)
            if st != 0:
                raise sg.SgemmError(st)

        kms, launches = timed_launches(torch, stream, launch)
        med = statistics.median(kms)
        flops, nbytes = algorithmic_flops(M, N, K), algorithmic_bytes(M, N, K)
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        _, m_main, n_main = sg.sgemm_f32_auto_plan(0, 0, M, N, K, cus)
        rec = {"config": name, "shape": [M, N, K], "dist": dist, "seed": seed,
               "algo": sg.sgemm_f32_algo_name(algo),
               "tile": sg.sgemm_f32_mfma_tile_name(sg.sgemm_f32_mfma_select(
                   m_main, n_main, K, cus)) if algo == sg.ALGO_MFMA else None,
               "blocks_cover": [m_main, n_main],
               "kernel_ms_median": round(med, 5), "kernel_ms_mean": round(sum(kms) / len(kms), 5),
               "kernel_ms_min": round(min(kms), 5), "launches": launches,
               "timing": "median, mean and minimum of 5 back-to-back runs' average",
               "tflops": round(flops / (med * 1e-3) / 1e12, 3),
               "pct_fp32_peak": round(100 * flops / (med * 1e-3) / 1e12 / PEAK_FP32_TFLOPS, 2),
               "gbs": round(nbytes / (med * 1e-3) / 1e9, 1),
               "pct_hbm_peak": round(100 * nbytes / (med * 1e-3) / 1e9 / PEAK_HBM_GBS, 2),
               "intensity_flop_per_byte": round(intensity(M, N, K), 2)}
        if name == "c4b":
            import synthgen
            bufs = [dB] + [torch.from_numpy(synthgen.matrix(K, N, seed=seed + 100 + i, stream=1,
                                                            dist=dist)).cuda() for i in range(4)]
            turn = [0]

            def rotated():
                launch(bufs[turn[0] % len(bufs)].data_ptr())
                turn[0] += 1
            rms, _ = timed_launches(torch, stream, rotated)
            rmed = statistics.median(rms)
            rec["rotated"] = {"b_buffers": len(bufs), "bytes": 4 * K * N * len(bufs),
                              "kernel_ms_median": round(rmed, 5),
                              "kernel_ms_min": round(min(rms), 5),
                              "gbs": round(nbytes / (rmed * 1e-3) / 1e9, 1),
                              "pct_hbm_peak": round(100 * nbytes / (rmed * 1e-3) / 1e9 /
                                                    PEAK_HBM_GBS, 2)}
            del bufs
        if algo == sg.ALGO_MFMA:
            sms, _ = timed_launches(torch, stream, lambda: _check(sg.sgemm_f32_algo(
                M, N, K, dA.data_ptr(), K, dB.data_ptr(), N, dC.data_ptr(), N, stream.cuda_stream,
                sg.ALGO_BF16X6), sg))
            rec["bf16x6"] = split_record(flops, statistics.median(sms))
        if args.cpu_seconds > 0:
            rec["host_blocked"] = cpu_blocked(A, B, M, N, K, reps=3 if M * N * K < 1e10 else 1)
        if name in ("c1", "c2") and args.cpu_seconds > 0:
            import oracle
            for threads in (1, host_threads()):
                t0 = time.perf_counter()
                oracle.sgemm(A[:, :K], B[:, :N], threads=threads)
                t = time.perf_counter() - t0
                rec[f"oracle_{'1' if threads == 1 else 'all'}_thread"] = {
                    "threads": threads, "ms": round(t * 1e3, 1),
                    "gflops": round(flops / t / 1e9, 3)}
        del dA, dB, dC
        print(json.dumps(rec), flush=True)
    print(json.dumps({"sclk_after": gpu_sclk(torch)}), flush=True)


# Shapes of the tile-choice model: the five workloads and nine others that mix
# wave quantisation, ragged edges, short and long k, and cached and uncached sizes.
TILE_SHAPES = [(8192, 8192, 8192), (2048, 3072, 4096), (4095, 4097, 1023), (1024, 1024, 1024),
               (512, 512, 512), (3000, 2000, 1500), (1000, 5000, 2000), (6000, 6000, 1000),
               (256, 8192, 8192), (8192, 256, 8192), (4096, 4096, 256), (16384, 16384, 1024),
               (2048, 2048, 2048), (4096, 4096, 4096), (128, 128, 65536), (512, 512, 32768),
               (256, 256, 16384), (512, 512, 4096), (1000, 1000, 8192)]


def tile_sweep(torch, sg, shapes, args):
    """Kernel time of every tile configuration of the matrix-core rung on each shape
    (one JSON line per shape and configuration)."""
    stream = torch.cuda.current_stream()
    ta, tb = (int(args.layout[0] == "T"), int(args.layout[1] == "T"))
    for (M, N, K) in shapes:
        _, _, dA, dB, dC = make_inputs(torch, M, N, K, args.seed, layout=(ta, tb))
        flops = algorithmic_flops(M, N, K)
        lda, ldb = (M if ta else K), (K if tb else N)

        def launch(tile):
            st = sg.sgemm_f32_ex_mfma_tile(ta, tb, M, N, K, 1.0, dA.data_ptr(), lda,
                                           dB.data_ptr(), ldb, 0.0, dC.data_ptr(), N,
                                           stream.cuda_stream, tile)
            if st != 0:
                raise sg.SgemmError(st, "sgemm_f32_ex_mfma_tile")

        def timed(tile, n, regions=1):
            """Per-region average kernel time of n back-to-back launches (ms)."""
            out = []
            for _ in range(regions):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                for _ in range(n):
                    launch(tile)
                b.record(stream)
                torch.cuda.synchronize()
                out.append(a.elapsed_time(b) / n)
            return out

        auto = sg.sgemm_f32_mfma_select(M, N, K, torch.cuda.get_device_properties(0)
                                        .multi_processor_count)
        # clocks settle on about half a second of work before the first timing
        est = max(timed(auto, 2)[-1], 1e-3)
        timed(auto, max(1, min(5000, int(500 / est))))
        for tile in range(sg.sgemm_f32_mfma_tiles()):
            est = max(min(timed(tile, 2)), 1e-3)
            timed(tile, max(2, min(2000, int(50 / est))))
            n = max(args.steps, min(2000, int(150 / est))) // 5 + 1
            kms = timed(tile, n, regions=5)
            avg = sum(kms) / len(kms)
            print(json.dumps({"shape": [M, N, K], "layout": args.layout, "tile": tile,
                              "name": sg.sgemm_f32_mfma_tile_name(tile), "chosen": tile == auto,
                              "kernel_ms_avg": round(avg, 5), "kernel_ms_min": round(min(kms), 5),
                              "tflops": round(flops / (avg * 1e-3) / 1e12, 2), "steps": 5 * n}),
                  flush=True)
        del dA, dB, dC


def main(argv=None):
    p = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=60)
    p.add_argument("--shape", default="8192,8192,8192", help="M,N,K of the timed product")
    p.add_argument("--algo", default="auto")
    p.add_argument("--seed", type=int, default=6)
    p.add_argument("--dist", default="normal", choices=["normal", "uniform_pm1", "smallint"],
                   help="distribution of the A and B entries")
    p.add_argument("--rotate", type=int, default=1,
                   help="rotate B over this many distinct buffers (5 x 64 MiB for 1x4096x4096 "
                        "exceeds the 256 MB Infinity Cache, so B comes from HBM)")
    p.add_argument("--no-also", action="store_true", help="skip the 2048x3072x4096 product")
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="CPU time budget of the oracle baseline (0 = skip)")
    p.add_argument("--floor", action="store_true",
                   help="time the smallest launches (K = 0, 1x1x1, one block and one k window of "
                        "the small tiles, one window on 256 blocks) back to back, one JSON line each")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a device copy of known size (for HBM counter calibration)")
    p.add_argument("--ladder", action="store_true",
                   help="time every algorithm of the ladder on --shape instead (one JSON line "
                        "per algorithm)")
    p.add_argument("--layout", default="NN", choices=["NN", "NT", "TN", "TT"],
                   help="storage order of A and B for the timed product (T: the operand is "
                        "passed transposed through sgemm_f32_ex)")
    p.add_argument("--configs", action="store_true",
                   help="report every workload (512^3, 1024^3, 2048x3072x4096, 4095x4097x1023, "
                        "1x4096x4096, 8192^3) instead, one JSON line each")
    p.add_argument("--workspace", action="store_true",
                   help="time sgemm_f32_ex_ws with the workspace sgemm_f32_workspace_size asks "
                        "for (split-k for products with few blocks of C)")
    p.add_argument("--tiles", action="store_true",
                   help="time every tile configuration of the matrix-core rung on --shape, or on "
                        "the tile-model shapes with --shape all (one JSON line per configuration)")
    args = p.parse_args(argv)

    if args.gpus != 1:
        print(json.dumps({"error": "the product runs on one GPU; sharding across GPUs is not implemented, so --gpus must be 1",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    import torch

    import dense_fp32_matrix_f32_amd as sg
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}), flush=True)
        sys.exit(1)
    sg.lib()

    if args.copy_calibration:
        n = 64 << 20  # 64 Mi floats = 256 MiB each way
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_each_way": 4 * n, "launches": 3}), flush=True)
        return

    if args.floor:
        launch_floor(torch, sg)
        return
    if args.configs:
        config_report(torch, sg, args)
        return
    if args.tiles:
        shapes = TILE_SHAPES if args.shape == "all" else \
            [tuple(int(x) for x in args.shape.split(","))]
        tile_sweep(torch, sg, shapes, args)
        return
    M, N, K = (int(x) for x in args.shape.split(","))
    if args.ladder:
        ladder(torch, sg, M, N, K, args)
        return
    algo = sg.ALGOS[args.algo]
    dist_name = {"normal": "N(0,1)", "uniform_pm1": "U[-1,1)", "smallint": "integers in [-4,4]"}
    print(f"[bench] generating {M}x{K} and {K}x{N} {dist_name[args.dist]} inputs (seed {args.seed})",
          file=sys.stderr, flush=True)
    layout = (int(args.layout[0] == "T"), int(args.layout[1] == "T"))
    A, B, dA, dB, dC = make_inputs(torch, M, N, K, args.seed, dist=args.dist, layout=layout)
    dBs = [dB]
    if args.rotate > 1:
        import synthgen
        ta_, tb_ = layout
        for r in range(1, args.rotate):
            dBs.append(torch.from_numpy(synthgen.matrix(N if tb_ else K, K if tb_ else N,
                                                        seed=args.seed + 100 + r, stream=1,
                                                        dist=args.dist)).cuda())
    # the algorithm the automatic choice takes for this shape and storage order
    chosen, _, _ = sg.sgemm_f32_auto_plan(layout[0], layout[1], M, N, K)
    used = chosen if algo == sg.ALGO_AUTO else algo
    print(f"[bench] timing {args.steps} steps after {args.warmup} warm-up, algo "
          f"{sg.sgemm_f32_algo_name(used)}", file=sys.stderr, flush=True)
    ws = None
    if args.workspace:
        nbytes = sg.sgemm_f32_workspace_size(layout[0], layout[1], M, N, K)
        ws = torch.empty(max(nbytes // 4, 1), dtype=torch.float32, device="cuda")
        print(f"[bench] workspace {nbytes} bytes (sgemm_f32_ex_ws)", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    sclk_before = gpu_sclk(torch)
    sclk_timed = []
    wall, kavg = time_product(torch, sg, M, N, K, dA, dBs, dC, algo, args.steps, args.warmup,
                              layout, workspace=ws, sclk_log=sclk_timed)
    sclk_after = gpu_sclk(torch)
    flops = algorithmic_flops(M, N, K)
    ms_per_step = wall * 1e3 / args.steps
    value = flops / (wall / args.steps) / 1e12
    achieved = flops / (kavg * 1e-3) / 1e12
    rec = {
        "metric": "SGEMM TFLOP/s (2MNK/t) + % FP32 peak at 2048\u00d74096\u00d73072 and 8192\u00b3",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "pct_fp32_peak": round(100 * value / PEAK_FP32_TFLOPS, 2),
        "config": {"workload": f"C=A*B fp32 row-major M={M} N={N} K={K}, A,B iid "
                               f"{dist_name[args.dist]} seed {args.seed}" +
                               ("" if layout == (0, 0) else f", operands {args.layout}") +
                               (f", B rotated over {args.rotate} buffers" if args.rotate > 1
                                else "") +
                               (f", split-k workspace {4 * ws.numel()} bytes" if ws is not None
                                else ""),
                   "M": M, "N": N, "K": K, "algo": sg.sgemm_f32_algo_name(used),
                   "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": PEAK_FP32_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP32_TFLOPS, 4),
                     "traffic": read_traffic() if (M, N, K, layout) == (8192, 8192, 8192, (0, 0))
                     else None,
                     "kernel_ms_avg": round(kavg, 4),
                     "algorithmic_flops": flops, "algorithmic_bytes": algorithmic_bytes(M, N, K),
                     "intensity_flop_per_byte": round(intensity(M, N, K), 2)},
        "sclk_smu_average_mhz": {"before": sclk_before,
                                 "timed": sclk_timed[0] if sclk_timed else None,
                                 "after": sclk_after,
                                 "note": "driver-reported running average (lags the kernel's "
                                         "clock); the kernel's clock is measured from counters"},
    }
    if used in (sg.ALGO_SKINNY, sg.ALGO_SKINNY_N):
        # few rows or columns: the product streams one operand, so HBM bounds it
        gbs = algorithmic_bytes(M, N, K) / (kavg * 1e-3) / 1e9
        rec["roofline"].update({"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                                "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4)})
    if layout == (0, 0) and algo == sg.ALGO_AUTO and M > 8 and N > 8:
        # the same product on the split-precision rung (fp32 accuracy on the bf16
        # matrix cores), reported beside the fp32 result, never as the value
        _, savg = time_product(torch, sg, M, N, K, dA, dB, dC, sg.ALGO_BF16X6, args.steps,
                               args.warmup)
        rec["bf16x6"] = split_record(flops, savg)
        rec["bf16x6"]["note"] = ("fp32 product on bf16 matrix cores, operands split into three "
                                 "bf16 parts (six part products), fp32 accumulation")
    del dA, dB, dC, dBs
    if not args.no_also:
        m2, n2, k2 = 2048, 3072, 4096
        print(f"[bench] timing {m2}x{n2}x{k2}", file=sys.stderr, flush=True)
        _, _, eA, eB, eC = make_inputs(torch, m2, n2, k2, 3)
        # A short product needs a time-based warm-up for the clocks to settle, and
        # enough timed launches to cover a few hundred milliseconds.
        est_ms = algorithmic_flops(m2, n2, k2) / 120e12 * 1e3
        warm2 = max(args.warmup, int(300 / est_ms))
        steps2 = max(args.steps, int(200 / est_ms))
        w2, k2avg = time_product(torch, sg, m2, n2, k2, eA, eB, eC, sg.ALGO_AUTO, steps2, warm2)
        f2 = algorithmic_flops(m2, n2, k2)
        rec["also"] = {"workload": f"C=A*B fp32 row-major M={m2} N={n2} K={k2}, N(0,1) seed 3",
                       "steps": steps2, "warmup": warm2,
                       "value": round(f2 / (w2 / steps2) / 1e12, 3), "unit": "TFLOP/s",
                       "kernel_tflops": round(f2 / (k2avg * 1e-3) / 1e12, 3),
                       "kernel_ms_avg": round(k2avg, 4),
                       "pct_fp32_peak": round(100 * f2 / (k2avg * 1e-3) / 1e12 / PEAK_FP32_TFLOPS, 2)}
        del eA, eB, eC
    if args.cpu_seconds > 0 and layout == (0, 0):
        print(f"[bench] oracle CPU baseline (~{args.cpu_seconds:.0f} s)", file=sys.stderr,
              flush=True)
        rec["cpu_baseline"] = cpu_baseline(A, B, M, N, K, args.cpu_seconds)
        print("[bench] blocked host SGEMM", file=sys.stderr, flush=True)
        rec["cpu_blocked"] = cpu_blocked(A, B, M, N, K)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()

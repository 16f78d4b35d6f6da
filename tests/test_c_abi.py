"""The boundary used from plain C: tests/c_abi/consumer.c includes only
include/sgemm_f32.h and links libsgemm_f32.so.  On the CPU it must compile and
link with warnings as errors; on the GPU its results (sgemm_f32, and the general
form with both operands transposed, alpha = 2, beta = -1) must equal the
oracle's bit for bit on small-integer data."""
import os
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _c_build():
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "c_abi_build", os.path.join(ROOT, "tests", "c_abi", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


CONSUMER = os.path.join(ROOT, "tests", "c_abi", "consumer")


def test_consumer_compiles_and_links():
    out = _c_build().build(os.path.join(ROOT, "tests", "c_abi", "consumer.check"))
    try:
        assert os.path.getsize(out) > 0
    finally:
        os.remove(out)


@pytest.mark.gpu
@pytest.mark.parametrize("shape", [(300, 257, 131), (2049, 4097, 100)],
                         ids=lambda s: "x".join(map(str, s)))
def test_consumer_matches_oracle(tmp_path, shape):
    import oracle
    import synthgen
    from gpu_helpers import log
    assert os.path.exists(CONSUMER), "tests/c_abi/consumer is not built (run __graft_entry__.build())"
    M, N, K = shape
    A = synthgen.matrix(M, K, seed=71, stream=0, dist="smallint")
    B = synthgen.matrix(K, N, seed=71, stream=1, dist="smallint")
    C0 = synthgen.matrix(M, N, seed=71, stream=2, dist="smallint")
    files = {n: str(tmp_path / f"{n}.bin") for n in ("a", "b", "c0", "c", "cex")}
    A.tofile(files["a"]); B.tofile(files["b"]); C0.tofile(files["c0"])
    log(f"[gpu] C consumer {M}x{N}x{K}")
    r = subprocess.run([CONSUMER, str(M), str(N), str(K), files["a"], files["b"], files["c0"],
                        files["c"], files["cex"]], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    C = np.fromfile(files["c"], dtype=np.float32).reshape(M, N)
    Cex = np.fromfile(files["cex"], dtype=np.float32).reshape(M, N)
    want, _ = oracle.sgemm(A, B)
    assert np.array_equal(C.astype(np.float64), want)
    want_ex, _ = oracle.sgemm_ex(A, B, False, False, 2.0, -1.0, C0)
    assert np.array_equal(Cex.astype(np.float64), want_ex)

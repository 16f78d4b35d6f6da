"""The benchmark's work and traffic formulas against the figures the pages print
(tests/golden/traffic_model.txt) and against closed forms."""
import pytest

import bench
from oracle_pins import read_golden


def test_traffic_counts_at_1024():
    g = read_golden("traffic_model.txt")
    n, tile = int(g["n"]), int(g["tile"])
    assert bench.naive_global_reads(n) == int(g["naive_reads"])
    assert bench.tiled_global_reads(n, tile) == int(g["tiled_reads"])


def test_intensity_figures():
    g = read_golden("traffic_model.txt")
    # naive: 2 flops per 2 loads of 4 bytes
    assert 2 / (2 * 4) == pytest.approx(float(g["naive_intensity"]))
    assert bench.tile_intensity(16, 16) == pytest.approx(float(g["tiled_intensity"]))
    d = int(g["square_intensity_divisor"])
    for n in (512, 1024, 8192):
        assert bench.intensity(n, n, n) == pytest.approx(n / d)


def test_work_and_bytes():
    assert bench.algorithmic_flops(2048, 3072, 4096) == 2 * 2048 * 3072 * 4096
    assert bench.algorithmic_bytes(2048, 3072, 4096) == 4 * (2048 * 4096 + 4096 * 3072 +
                                                              2048 * 3072)
    # row times matrix: about half a flop per byte, far below the ridge point
    assert bench.intensity(1, 4096, 4096) == pytest.approx(0.4998, abs=1e-4)


def test_multi_gpu_request_is_refused(capsys):
    with pytest.raises(SystemExit) as e:
        bench.main(["--gpus", "2"])
    assert e.value.code == 2
    assert "one GPU" in capsys.readouterr().out

"""The CPU oracle against facts fixed by the pages and by mathematics (no GPU)."""
import numpy as np
import pytest

import oracle
from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(oracle.load())


def test_acceptance_rule():
    C = np.array([1.0, 2.0, 0.0, np.inf, np.nan])
    S = np.array([1.0, 10.0, 0.0, 1.0, 1.0])
    # inside the bound, on it, beyond it
    assert oracle.accept(np.array([1.0 + 4e-4]), C[:1], S[:1])
    assert not oracle.accept(np.array([1.0 + 6e-4]), C[:1], S[:1])
    assert oracle.accept(np.array([2.0 + 4.9e-3]), C[1:2], S[1:2])
    # near-zero results are judged by the absolute term
    assert oracle.accept(np.array([9e-7]), C[2:3], S[2:3])
    assert not oracle.accept(np.array([2e-6]), C[2:3], S[2:3])
    # a NaN from the GPU is never accepted against a finite value
    assert not oracle.accept(np.array([np.nan]), C[:1], S[:1])
    # matching non-finite values are accepted
    assert oracle.accept(np.array([np.inf]), C[3:4], S[3:4])


def test_rejects_bad_arguments():
    A = np.zeros((3, 4), dtype=np.float32)
    B = np.zeros((5, 2), dtype=np.float32)
    with pytest.raises(ValueError):
        oracle.sgemm(A, B)
    with pytest.raises(ValueError):
        oracle.sgemm_elems(A, np.zeros((4, 2), np.float32), [3], [0])

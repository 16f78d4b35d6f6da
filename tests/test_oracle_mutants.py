"""Planted mistakes in the CPU oracle must each fail at least one pin.

Each case copies the oracle's C source, changes one expression into a plausible
mistake (a dropped term, a wrong sign, a transposed operand, a wrong index, a
narrower accumulator), compiles it on the CPU and runs the pins against it.
"""
import os

import pytest

import oracle
from oracle_pins import ALL_PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "sgemm_oracle.c")

MUTANTS = {
    "drop_last_term": ("for (int64_t k = 0; k < K; ++k) {", "for (int64_t k = 0; k < K - 1; ++k) {"),
    "skip_first_term": ("for (int64_t k = 0; k < K; ++k) {", "for (int64_t k = 1; k < K; ++k) {"),
    "wrong_sign": ("c += a * b;", "c -= a * b;"),
    "transposed_B": ("double b = (double)B[k * ldb + j];", "double b = (double)B[j * ldb + k];"),
    "transposed_A": ("double a = (double)A[i * lda + k];", "double a = (double)A[k * lda + i];"),
    "a_index_uses_j": ("double a = (double)A[i * lda + k];", "double a = (double)A[j * lda + k];"),
    "float_accumulator": ("double c = 0.0;", "float c = 0.0f;"),
    "scale_without_abs": ("s += fabs(a) * fabs(b);", "s += a * b;"),
    "nonzero_start": ("double c = 0.0;", "double c = 1e-300 + (K == 0);"),
    "b_uses_lda": ("double b = (double)B[k * ldb + j];", "double b = (double)B[k * lda + j];"),
}


def _mutant_lib(tmp_path, name):
    before, after = MUTANTS[name]
    text = open(SRC, encoding="utf-8").read()
    assert text.count(before) == 1, f"pattern for {name} not found exactly once"
    src = tmp_path / f"{name}.c"
    src.write_text(text.replace(before, after), encoding="utf-8")
    lib = tmp_path / f"lib{name}.so"
    oracle.build(force=True, src=str(src), out=str(lib))
    return oracle.load(str(lib))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(tmp_path, name):
    lib = _mutant_lib(tmp_path, name)
    failed = []
    for pin in ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError):
            failed.append(pin.__name__)
    assert failed, f"no pin caught the planted mistake {name}"

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
    "wrong_sign": ("\n        c += a * b;", "\n        c -= a * b;"),
    "transposed_B": ("double b = (double)B[k * ldb + j];", "double b = (double)B[j * ldb + k];"),
    "transposed_A": ("double a = (double)A[i * lda + k];", "double a = (double)A[k * lda + i];"),
    "a_index_uses_j": ("double a = (double)A[i * lda + k];", "double a = (double)A[j * lda + k];"),
    "float_accumulator": ("\n    double c = 0.0;\n    double s = 0.0;\n    for",
                          "\n    float c = 0.0f;\n    double s = 0.0;\n    for"),
    "scale_without_abs": ("\n        s += fabs(a) * fabs(b);", "\n        s += a * b;"),
    "nonzero_start": ("\n    double c = 0.0;\n    double s = 0.0;\n    for",
                      "\n    double c = 1e-300 + (K == 0);\n    double s = 0.0;\n    for"),
    "b_uses_lda": ("double b = (double)B[k * ldb + j];", "double b = (double)B[k * lda + j];"),
    # the general form
    "ex_transa_ignored": ("p->transa ? (double)p->A[k * p->lda + i]",
                          "p->transa ? (double)p->A[i * p->lda + k]"),
    "ex_transb_ignored": ("p->transb ? (double)p->B[j * p->ldb + k]",
                          "p->transb ? (double)p->B[k * p->ldb + j]"),
    "ex_transb_reversed_k": ("p->transb ? (double)p->B[j * p->ldb + k]",
                             "p->transb ? (double)p->B[j * p->ldb + (p->K - 1 - k)]"),
    "ex_beta_read_when_zero": ("if (p->beta != 0.0) {", "if (1) {"),
    "ex_alpha_zero_reads_ab": ("if (p->alpha != 0.0) {", "if (1) {"),
    "ex_alpha_on_c": ("out += p->beta * cin;", "out += p->alpha * p->beta * cin;"),
    "ex_beta_sign": ("out += p->beta * cin;", "out -= p->beta * cin;"),
    "ex_scale_without_beta": ("scale += fabs(p->beta) * fabs(cin);", "scale += 0.0 * fabs(cin);"),
    "ex_alpha_dropped": ("double out = p->alpha * c;", "double out = c;"),
    "ex_wrong_sign": ("\n            c += a * b;", "\n            c -= a * b;"),
    "ex_scale_without_abs": ("\n            s += fabs(a) * fabs(b);", "\n            s += a * b;"),
    # the general form's leading dimensions: a row length read in place of ld
    "ex_a_uses_k_for_lda": ("(double)p->A[i * p->lda + k]", "(double)p->A[i * p->K + k]"),
    "ex_at_uses_m_for_lda": ("(double)p->A[k * p->lda + i]", "(double)p->A[k * p->M + i]"),
    "ex_b_uses_n_for_ldb": ("(double)p->B[k * p->ldb + j]", "(double)p->B[k * p->N + j]"),
    "ex_bt_uses_k_for_ldb": ("(double)p->B[j * p->ldb + k]", "(double)p->B[j * p->K + k]"),
    "ex_cin_uses_n_for_ldcin": ("p->Cin[i * p->ldcin + j]", "p->Cin[i * p->N + j]"),
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

"""The torch helper's reading of tensor strides (host logic, no GPU)."""
import pytest

import dense_fp32_matrix_f32_amd as sg


@pytest.mark.parametrize("rows,cols,s0,s1,want", [
    (5, 4, 4, 1, (4, False)),     # dense row-major
    (5, 4, 9, 1, (9, False)),     # row-major view with padded rows
    (5, 4, 1, 5, (5, True)),      # X.t() of a dense 4 x 5 array
    (5, 4, 1, 8, (8, True)),      # transpose of a padded array
    (1, 4, 0, 1, (4, False)),     # one row: its row stride is never used
    (3, 1, 1, 1, (1, False)),     # one column, dense
    (3, 1, 7, 3, (7, False)),     # one column of a wider array
    (1, 4, 1, 3, (3, True)),      # one row with a stride along it: a K x 1 stored column
    (0, 4, 0, 1, (4, False)),     # empty
])
def test_layout_accepts(rows, cols, s0, s1, want):
    assert sg._layout(rows, cols, s0, s1, "X") == want


@pytest.mark.parametrize("rows,cols,s0,s1", [
    (5, 4, 0, 1),   # X.expand(5, 4) of one row
    (5, 1, 0, 1),   # X.expand(5, 1) of one element
    (5, 4, 1, 0),   # expanded along columns, then seen as a transpose
    (1, 4, 1, 0),   # one element repeated along a row
    (5, 4, 2, 1),   # overlapping rows (as_strided)
    (5, 4, 1, 3),   # overlapping columns of a transposed view
    (5, 4, 3, 2),   # no unit stride
])
def test_layout_rejects_broadcast_and_overlap(rows, cols, s0, s1):
    with pytest.raises(ValueError):
        sg._layout(rows, cols, s0, s1, "X")

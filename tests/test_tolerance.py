"""The GPU parity bound is applied row by row (CPU test of the comparison
helper the GPU tests use): |got[r, i] - want[r, i]| <= 1e-2 max(1, max_j
|want[r, j]|), so a large output loosens the bound of its own row only, and
rows of unit scale keep the absolute bound whatever the other rows hold."""
import numpy as np
import pytest

from _gpu import MAX_ABS, assert_close, scaled_max_abs


def _rows(*rows):
    return np.array([list(r) * 16 for r in rows], dtype=np.float64)  # [rows, 64]


def test_small_rows_keep_the_absolute_bound_next_to_a_large_row():
    want = _rows([0.1, 0.2, -0.3, 0.05], [9.0, 0.3, -4.0, 1.0])
    got = want.copy()
    got[0, 1] += 0.02  # 2e-2 in a unit-scale row: out of bounds whatever row 1 holds
    assert scaled_max_abs(got, want) == pytest.approx(0.02)
    with pytest.raises(AssertionError, match="max abs"):
        assert_close(got, want, "x")


def test_elements_of_a_large_row_share_its_allowance():
    want = _rows([0.1, 0.2, -0.3, 0.05], [9.0, 0.3, -4.0, 1.0])
    got = want.copy()
    got[1, 1] += 0.05  # 0.05 on an element of 0.3 in a row of scale 9: within 1e-2 * 9
    max_abs, _ = assert_close(got, want, "x")
    assert max_abs == pytest.approx(0.05 / 9.0)
    assert max_abs <= MAX_ABS
    got[1, 1] += 0.05  # 0.1 > 0.09: out of bounds
    with pytest.raises(AssertionError, match="max abs"):
        assert_close(got, want, "x")


def test_one_dimensional_arrays_scale_per_element():
    want = np.array([9.0, 0.1, 0.2] * 100)
    got = want.copy()
    got[1] += 0.02
    assert scaled_max_abs(got, want) == pytest.approx(0.02)


def test_relative_l2_is_checked_too():
    want = np.full((10, 100), 0.5)
    got = want + 0.004  # within max abs, but rel L2 = 8e-3 > 5e-3
    with pytest.raises(AssertionError, match="relative L2"):
        assert_close(got, want, "x")

"""The parity checker of the GPU tests must be able to fail: an output row the
kernel never wrote (left at the NaN it was filled with), a NaN or infinity
where the oracle is finite, and a row the oracle did not compute all count as
an infinite error.  CPU only."""
import math

import numpy as np

from gpu_util import all_rows_written, max_err


def test_unwritten_row_fails():
    ref = np.zeros((4, 3, 8))
    gpu = np.zeros((4, 3, 8), np.float32)
    gpu[2, 1, :] = np.nan
    assert max_err(gpu, ref) == math.inf
    assert not all_rows_written(gpu)


def test_single_nan_value_fails():
    ref = np.ones((2, 16))
    gpu = np.ones((2, 16), np.float32)
    gpu[1, 7] = np.nan
    assert max_err(gpu, ref) == math.inf


def test_gpu_infinity_fails():
    ref = np.ones((3, 4))
    gpu = np.ones((3, 4), np.float32)
    gpu[0, 0] = np.inf
    assert max_err(gpu, ref) == math.inf


def test_row_the_oracle_skipped_fails():
    """A selected row that the oracle left at NaN (not computed) is an error
    in the test itself, not a pass."""
    ref = np.full((4, 8), np.nan)
    ref[0] = 0.5
    gpu = np.full((4, 8), 0.5, np.float32)
    assert max_err(gpu, ref, rows=[0]) == 0.0
    assert max_err(gpu, ref, rows=[0, 1]) == math.inf


def test_rows_are_chosen_by_index():
    ref = np.zeros((3, 5))
    gpu = np.zeros((3, 5), np.float32)
    gpu[1] = 0.25
    gpu[2] = np.nan
    assert max_err(gpu, ref, rows=[0]) == 0.0
    assert max_err(gpu, ref, rows=[1]) == 0.25
    assert max_err(gpu, ref, rows=[0, 2]) == math.inf


def test_empty_list_lse_agrees():
    """-inf on both sides (the lse of an empty list) is agreement; -inf on one
    side only is not."""
    ref = np.array([[-np.inf, 1.0]])
    gpu = np.array([[-np.inf, 1.0]], np.float32)
    assert max_err(gpu, ref) == 0.0
    assert max_err(np.array([[0.0, 1.0]], np.float32), ref) == math.inf
    assert max_err(gpu, np.array([[0.0, 1.0]])) == math.inf


def test_one_dimensional_arrays_are_rows_of_one():
    ref = np.array([1.0, 2.0, 3.0])
    gpu = np.array([1.0, 2.5, np.nan], np.float32)
    assert max_err(gpu, ref, rows=[0, 1]) == 0.5
    assert max_err(gpu, ref) == math.inf


def test_plain_difference():
    rng = np.random.default_rng(0)
    ref = rng.standard_normal((5, 6, 7))
    gpu = (ref + 1e-4).astype(np.float32)
    assert abs(max_err(gpu, ref) - 1e-4) < 1e-6


def test_size_mismatch_is_an_error():
    import pytest
    with pytest.raises(ValueError):
        max_err(np.zeros((2, 3)), np.zeros((2, 4)))

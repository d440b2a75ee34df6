"""The same-path comparison helper of the GPU tests: one bf16 step at the
element's magnitude, never less than SAME_ABS."""
import numpy as np

from tests._util import SAME_ABS, same_path_excess


def test_one_bf16_step_allowed():
    # bf16 steps: 2^-6 in [2, 4), 2^-8 in [0.5, 1), 2^-3 in [16, 32)
    assert same_path_excess([3.0], [3.0 + 2.0 ** -6]) <= 0
    assert same_path_excess([3.0], [3.0 + 2.0 ** -5]) > 0
    assert same_path_excess([20.0], [20.0 - 2.0 ** -3]) <= 0
    assert same_path_excess([20.0], [20.0 - 2.0 ** -2]) > 0


def test_floor_is_same_abs():
    assert same_path_excess([0.5], [0.5 + 0.9 * SAME_ABS]) <= 0
    assert same_path_excess([0.5], [0.5 + 1.1 * SAME_ABS]) > 0
    assert same_path_excess(np.zeros(4), np.zeros(4)) <= 0

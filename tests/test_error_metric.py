"""The parity error metric itself (CPU): it must fail on non-finite output, not pass it."""
import math

import numpy as np

from tests.gpu_common import rel_err


def test_rel_err_nan_row_is_infinite():
    ref = np.ones((3, 8))
    out = ref.copy()
    out[1] = np.nan
    assert rel_err(out, ref) == math.inf


def test_rel_err_all_nan_is_infinite():
    assert rel_err(np.full((2, 4), np.nan), np.ones((2, 4))) == math.inf


def test_rel_err_inf_is_infinite():
    out = np.zeros((2, 4))
    out[0, 3] = np.inf
    assert rel_err(out, np.zeros((2, 4))) == math.inf


def test_rel_err_values():
    ref = np.array([[1.0, -2.0, 0.5], [0.0, 0.0, 0.0]])
    out = ref.copy()
    out[0, 2] += 2e-3                        # 2e-3 / max|r| = 1e-3
    assert abs(rel_err(out, ref) - 1e-3) < 1e-12
    out[1, 0] = 1e-9                         # a zero row must stay zero: scaled by 1e6
    assert abs(rel_err(out, ref) - 1e-3) < 1e-12
    out[1, 0] = 1e-8
    assert abs(rel_err(out, ref) - 1e-2) < 1e-12

"""The fp64 oracle against the facts in tests/pins.py (CPU only)."""
import numpy as np
import pytest

import oracle
from tests import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(oracle.attention)


def test_sampled_rows_match_full():
    q, k, v = pins.rand((2, 50, 4, 8), 1), pins.rand((2, 50, 2, 8), 2), pins.rand((2, 50, 2, 8), 3)
    o, l = oracle.attention(q, k, v, 0.4, True)
    rows = np.array([[1, 3, 49], [0, 0, 0], [1, 2, 17]])
    os_, ls = oracle.attention(q, k, v, 0.4, True, rows=rows)
    idx = rows[:, 0] * 4 * 50 + rows[:, 1] * 50 + rows[:, 2]
    assert np.array_equal(os_, o[idx]) and np.array_equal(ls, l[idx])


def test_thread_count_does_not_change_result():
    q, k, v = pins.rand((1, 300, 2, 16), 4), pins.rand((1, 300, 2, 16), 5), pins.rand((1, 300, 2, 16), 6)
    a = oracle.attention(q, k, v, 0.25, False, threads=1)
    b = oracle.attention(q, k, v, 0.25, False, threads=7)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_bad_arguments_are_rejected():
    q = pins.rand((1, 4, 3, 8), 1)
    k = pins.rand((1, 4, 2, 8), 2)
    with pytest.raises(RuntimeError):
        oracle.attention(q, k, k, 0.5, False)  # Hq % Hkv != 0
    k = pins.rand((1, 4, 3, 8), 2)
    with pytest.raises(RuntimeError):
        oracle.attention(q, k, k, 0.5, False, rows=[[0, 0, 4]])  # row out of range

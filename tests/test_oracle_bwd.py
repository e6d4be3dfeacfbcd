"""The fp64 backward oracle against the facts in tests/pins.py (CPU only)."""
import numpy as np
import pytest

import oracle
from tests import pins


@pytest.mark.parametrize("pin", pins.BWD_PINS, ids=lambda p: p.__name__)
def test_bwd_oracle_pin(pin):
    pin(oracle.attention, oracle.attention_bwd)


def test_bwd_groups_subset_and_threads():
    q, k, v = pins.rand((2, 40, 4, 8), 1), pins.rand((2, 30, 2, 8), 2), pins.rand((2, 30, 2, 8), 3)
    do = pins.rand((2, 40, 4, 8), 4)
    full = oracle.attention_bwd(q, k, v, do, 0.3, True)
    part = oracle.attention_bwd(q, k, v, do, 0.3, True, groups=[[1, 0], [0, 1]], threads=3)
    for a, b in zip(full, part):
        assert np.allclose(a[[2, 1]], b, atol=1e-14, rtol=0)


def test_bwd_bad_arguments():
    q = pins.rand((1, 4, 2, 8), 1)
    k = pins.rand((1, 4, 2, 8), 2)
    with pytest.raises(RuntimeError):
        oracle.attention_bwd(q, k, k, q, 0.5, False, groups=[[0, 2]])
    with pytest.raises(ValueError):
        oracle.attention_bwd(q, k, k, k[:, :3], 0.5, False)

"""The CPU oracle against closed forms, invariants and exact brute force (no GPU)."""

import pytest


import oracle
from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(oracle.default())


def test_oracle_rejects_bad_arguments():
    import numpy as np
    u = np.zeros((4, 4), np.float32)
    with pytest.raises(ValueError):
        oracle.jacobi(np.zeros((2, 4), np.float32), 1)
    with pytest.raises(ValueError):
        oracle.jacobi(u, -1)
    with pytest.raises(ValueError):
        oracle.jacobi(u, 5, checkpoints=[3, 1])
    with pytest.raises(ValueError):
        oracle.jacobi(u, 5, checkpoints=[6])
    with pytest.raises(ValueError):
        oracle.jacobi(u, 1, f=np.ones((4, 4), np.float32), h=0.0)


def test_zero_sweeps_is_identity():
    import numpy as np
    rng = np.random.default_rng(0)
    u = rng.standard_normal((9, 11))
    out, _ = oracle.jacobi(u, 0)
    assert np.array_equal(out, u)

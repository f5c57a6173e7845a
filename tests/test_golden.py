"""The stored oracle results of the 4096^2 and 8192^2 workloads hold together:
their row hashes follow the convention the GPU tests use, checked on rows whose
values are known without the oracle (ring rows, rows the top edge has not
reached after 2,000 sweeps, the top edge itself) and on the stored middle row."""

import json
import os

import numpy as np
import pytest

import make_golden

GOLDEN = os.path.dirname(make_golden.__file__)


def _load(name):
    return json.load(open(os.path.join(GOLDEN, f"{name}.json")))


def test_laplace4096_row_hashes():
    g = _load("laplace4096")
    nx = ny = 4096
    rows = g["row_sha256_16"]
    assert len(rows) == ny
    zero = make_golden.row_hashes(np.zeros((1, nx), np.float32))[0][0]
    one = make_golden.row_hashes(np.ones((1, nx), np.float32))[0][0]
    # more than 2000 rows below the top edge nothing has moved after 2000 sweeps
    assert all(h == zero for h in rows[: ny - 1 - g["sweeps"]])
    assert rows[ny - 1] == one
    assert rows[ny - 2] not in (zero, one)


def test_poisson8192_row_hashes():
    g = _load("poisson8192")
    nx = ny = 8192
    rows = g["row_sha256_16"]
    assert len(rows) == ny
    zero = make_golden.row_hashes(np.zeros((1, nx), np.float64))[0][0]
    assert rows[0] == zero and rows[ny - 1] == zero  # the zero Dirichlet ring
    mid = np.array([float.fromhex(v) for v in g["row"]], np.float64)[None, :]
    assert make_golden.row_hashes(mid)[0][0] == rows[g["row_index"]]
    assert len(set(rows[1:-1])) == ny - 2  # noisy source: no two interior rows alike


@pytest.mark.parametrize("dtype", [np.float32, np.float64])
def test_row_hash_is_byte_order_fixed(dtype):
    x = np.arange(12, dtype=dtype).reshape(3, 4)
    a, whole = make_golden.row_hashes(x)
    b, whole_be = make_golden.row_hashes(x.astype(np.dtype(dtype).newbyteorder(">")))
    assert a == b and whole == whole_be

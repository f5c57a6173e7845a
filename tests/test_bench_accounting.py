"""The byte accounting of bench.py's roofline mirrors how the persistent kernel
splits a streaming task into passes (deep passes, the shallow last pass that also
sums the residual, red-black passes) and which RESIDUAL tasks read the field.
Expected values are worked out by hand from that rule. No GPU needed."""

import os
import sys
import types

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


@pytest.mark.parametrize("n,depth,rb,want", [
    (50, 12, False, [12, 12, 12, 12, 2]),
    (12, 12, False, [4, 8]),
    (23, 12, False, [12, 8, 3]),
    (24, 12, False, [12, 4, 8]),
    (10, 12, False, [8, 2]),
    (8, 12, False, [8]),
    (7, 12, False, [7]),
    (14, 12, True, [8, 6]),
    (50, 8, False, [8, 8, 8, 8, 8, 8, 2]),
    (5, 1, False, [1, 1, 1, 1, 1]),
    (0, 12, False, []),
])
def test_pass_depths(n, depth, rb, want):
    got = bench.pass_depths(n, depth, rb)
    assert got == want
    assert sum(got) == n
    assert all(k in (1, 2, 3, 4, 5, 6, 7, 8, 12) for k in got)
    if got:
        assert got[-1] <= bench.SHALLOW_PASS


def _shape_only(nx, ny, dtype, poisson, script=()):
    """What the accounting reads of a workload: shape, type, source, script."""
    return types.SimpleNamespace(nx=nx, ny=ny, dtype=dtype, f=(object() if poisson else None),
                                 script=list(script))


def test_default_depth_follows_the_infinity_cache():
    # 8192^2 fp64 Poisson streams 3 x 512 MiB: deep passes; 4096^2 fp32 Laplace
    # streams 2 x 64 MiB, which the 256 MiB cache holds
    assert bench.default_depth(_shape_only(8192, 8192, np.float64, True)) == 12
    assert bench.default_depth(_shape_only(4096, 4096, np.float32, False)) == 8
    assert bench.default_depth(_shape_only(6000, 6000, np.float32, True)) == 12  # 3 x 137 MiB


def test_script_counts_fused_residuals():
    # the 8192^2 script: RESIDUAL; 10 x (SWEEP 50, RESIDUAL): only the first
    # residual reads the field, the others were summed by the pass before them
    script = [("residual",)] + [("sweep", 50), ("residual",)] * 10 + [("readback",)]
    w = _shape_only(8192, 8192, np.float64, True, script)
    assert bench.script_counts(w, 12, fuse=False) == (500, 50, 1)
    assert bench.script_counts(w, 8) == (500, 70, 1)
    # one pass per sweep (launch-style plans) fuses nothing
    assert bench.script_counts(w, 1) == (500, 500, 11)
    # red-black tasks and empty sweeps leave the next residual to read the field
    w = _shape_only(64, 64, np.float32, False,
                    [("sweep", 9), ("residual",), ("sweep_rb", 3), ("residual",), ("sweep", 0), ("residual",)])
    assert bench.script_counts(w, 8) == (12, 2 + 1, 2)


def test_script_counts_fused_tails():
    """fp64 at depth 12: a SWEEP task's last t <= 12 sweeps run on into the next
    SWEEP task when a RESIDUAL and a long enough SWEEP follow. The 8192^2 script's
    ten 50-sweep tasks: 12 x 4 and a fused tail of 2 (5 passes), then 40, 42, 44,
    46 sweeps left (12 x 3 and a fused tail each), 48 (12 x 3, then its last 12 as
    a pass of their own and the next task's first 12 summing the residual of level
    0: 5 passes), 38, 40, 42, and the last, 44 with nothing to fuse into (12 x 3,
    then 8 that sums the residual). The step's first RESIDUAL (of a field no pass
    has summed) runs the first task's first pass and sums its level 0, so that task
    starts 12 sweeps ahead: 42 passes for 500 sweeps and no pass that only reads."""
    script = [("residual",)] + [("sweep", 50), ("residual",)] * 10 + [("readback",)]
    w = _shape_only(8192, 8192, np.float64, True, script)
    assert bench.fuses(w, 12) and not bench.fuses(w, 8)
    stats = {}
    assert bench.script_counts(w, 12, stats=stats) == (500, 42, 0)
    assert stats["fused"] == 10
    # the same script in fp32 runs every task on its own
    w32 = _shape_only(8192, 8192, np.float32, True, script)
    assert not bench.fuses(w32, 12)
    assert bench.script_counts(w32, 12) == (500, 50, 1)
    # a next task shorter than the rest of the pass, and a red-black task next, do not
    # fuse: 30 -> 12, 12 and a tail of 6, which would need a SWEEP of at least 6 next
    # (5 is too short: the tail runs alone and sums the residual); 5 -> 5; 20 -> 12,
    # then its tail of 8 runs on 4 sweeps into the next 30 -> 26 left -> 12, 12 and a
    # tail of 2 (a red-black task follows); the red-black task -> one pass
    script = [("sweep", 30), ("residual",), ("sweep", 5), ("residual",), ("sweep", 20), ("residual",),
              ("sweep", 30), ("residual",), ("sweep_rb", 2), ("residual",)]
    w = _shape_only(300, 514, np.float64, True, script)
    sweeps, passes, reads = bench.script_counts(w, 12)
    assert sweeps == 87
    assert passes == 3 + 1 + 2 + 3 + 1
    assert reads == 1  # only the residual after the red-black task reads the field

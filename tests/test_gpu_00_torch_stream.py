"""PyTorch as plumbing: the engine on a torch-created stream (GPU).

Collected before the other GPU tests on purpose: the check runs in a child
process, and a process that already holds a cooperative (persistent) launch
context on the device makes the child's cooperative launch fail. The child
imports torch before loading the engine library so that both share torch's HIP
runtime (torch bundles its own copy).
"""

import pytest

from parity import say

pytestmark = pytest.mark.gpu


TORCH_STREAM_SCRIPT = r"""
import sys
import numpy as np
import torch                      # first: the process then has torch's HIP runtime,
sys.path.insert(0, sys.argv[1])   # and the engine library binds to the same one
import oracle
from iterative_stencil_pde_amd import inputs, pk
s = torch.cuda.Stream()
w = inputs.poisson_uniform(256, 0)
with pk.Engine(w.u0, w.f, h=w.h, mode=pk.PK_LAUNCH, stream=s.cuda_stream) as e:
    e.sweep(100)
    r = e.residual()
    got = e.readback()
for lay in (pk.PK_LAYOUT_STREAM, pk.PK_LAYOUT_AUTO):
    try:
        with pk.Engine(w.u0, w.f, h=w.h, stream=s.cuda_stream, layout=lay) as e:
            i = e.info()
            print("persistent on torch stream: layout", i.layout, "grid", i.grid_blocks,
                  "lds", i.lds_bytes, "occ", i.blocks_per_cu_max, flush=True)
            e.sweep(100)
            r2 = e.residual()
            got2 = e.readback()
    except pk.PkError as ex:
        print("persistent layout", lay, "failed:", ex, flush=True)
        raise
ref, res = oracle.jacobi(w.u0, 100, f=w.f, h=w.h, checkpoints=[100])
assert np.array_equal(got, ref) and np.array_equal(got2, ref)
assert abs(r - res[0]) <= 1e-9 * res[0] and r == r2
x = torch.arange(10, device="cuda", dtype=torch.float32)
assert float(x.sum()) == 45.0
print("torch stream ok", r)
"""


def test_engine_on_a_torch_stream():
    """PyTorch provides the stream (plumbing only); the engine's kernels run on it."""
    import os
    import subprocess
    import sys
    pytest.importorskip("torch")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, PK_DEBUG="1")
    out = subprocess.run([sys.executable, "-c", TORCH_STREAM_SCRIPT, root], capture_output=True,
                         text=True, timeout=300, env=env)
    say(out.stdout[-2000:] + out.stderr[-2000:])
    assert out.returncode == 0 and "torch stream ok" in out.stdout

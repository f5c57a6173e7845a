"""The entry point that allocates nothing (pk_sweep_noalloc) against the one it
is a variant of: a PK_LAUNCH engine running SWEEP n and RESIDUAL. Same kernels,
same grid, so the field and the residual must be equal bit for bit. Two calls in
a row on the library's per-GPU scratch, the second with a smaller input; the
device buffers come from the HIP runtime the library itself uses (the test
allocates, the entry point does not)."""

import ctypes

import numpy as np
import pytest

from iterative_stencil_pde_amd import inputs, pk
from parity import say

pytestmark = pytest.mark.gpu

HIP_MEMCPY_H2D, HIP_MEMCPY_D2H = 1, 2


class Hip:
    """The few runtime calls the test needs, from the runtime the engine library loaded."""

    def __init__(self):
        pk.load()
        self.rt = ctypes.CDLL("libamdhip64.so.7")
        self.rt.hipMalloc.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_size_t]
        self.rt.hipFree.argtypes = [ctypes.c_void_p]
        self.rt.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
        self.rt.hipStreamSynchronize.argtypes = [ctypes.c_void_p]

    def alloc(self, nbytes):
        p = ctypes.c_void_p()
        assert self.rt.hipMalloc(ctypes.byref(p), nbytes) == 0
        return p.value

    def put(self, dptr, a):
        assert self.rt.hipMemcpy(dptr, a.ctypes.data, a.nbytes, HIP_MEMCPY_H2D) == 0

    def get(self, dptr, a):
        assert self.rt.hipMemcpy(a.ctypes.data, dptr, a.nbytes, HIP_MEMCPY_D2H) == 0
        return a

    def sync(self):
        assert self.rt.hipStreamSynchronize(None) == 0

    def free(self, *ptrs):
        for p in ptrs:
            self.rt.hipFree(p)


def pitched(a, pitch):
    out = np.zeros((a.shape[0], pitch), a.dtype)
    out[:, : a.shape[1]] = a
    return out


def engine_reference(u, f, h, n):
    """SWEEP n, RESIDUAL, readback on a PK_LAUNCH engine with default options."""
    with pk.Engine(u, f, h=h, mode=pk.PK_LAUNCH) as e:
        e.sweep(n)
        r = e.residual()
        info = e.info()
        return e.readback(), r, info


def run_noalloc(hip, u, f, h, n, pitch):
    ny, nx = u.shape
    dt = pk.PK_F64 if u.dtype == np.float64 else pk.PK_F32
    nbytes = ny * pitch * u.dtype.itemsize
    d_u0, d_u1, d_r = hip.alloc(nbytes), hip.alloc(nbytes), hip.alloc(8)
    d_b = None
    try:
        up = pitched(u, pitch)
        hip.put(d_u0, up)
        hip.put(d_u1, up)  # both buffers carry the ring
        if f is not None:
            # the scaled source exactly as the engine forms it: (T)((h*h) * f)
            b = (np.float64(h) * np.float64(h) * f.astype(np.float64)).astype(u.dtype)
            d_b = hip.alloc(nbytes)
            hip.put(d_b, pitched(b, pitch))
        rc = pk.pk_sweep_noalloc(dt, nx, ny, pitch, d_u0, d_u1, d_b, n, d_r, None)
        assert rc == pk.PK_OK, pk.pk_strerror(rc)
        hip.sync()
        out = hip.get(d_u1 if n & 1 else d_u0, np.empty((ny, pitch), u.dtype))[:, :nx]
        r = hip.get(d_r, np.empty(1, np.float64))[0]
        return np.ascontiguousarray(out), float(r)
    finally:
        hip.free(d_u0, d_u1, d_r, *([d_b] if d_b else []))


def test_noalloc_matches_the_launch_engine_twice():
    hip = Hip()
    cases = [
        # (shape, dtype, poisson, sweeps): the second call is the smaller input
        ((257, 255), np.float32, True, 37),
        ((67, 131), np.float64, False, 12),
    ]
    for (ny, nx), dt, pois, n in cases:
        u = inputs.uniform(ny * 1000 + nx, 0, ny * nx, -1, 1).reshape(ny, nx).astype(dt)
        f = inputs.uniform(ny * 1000 + nx, 1, ny * nx, -20, 20).reshape(ny, nx).astype(dt) if pois else None
        h = 0.013
        ref, r_ref, info = engine_reference(u, f, h, n)
        got, r = run_noalloc(hip, u, f, h, n, info.pitch)
        nonbit = int(np.count_nonzero(got != ref))
        say(f"  {ny}x{nx} {np.dtype(dt).name} poisson={pois} n={n} grid={info.grid_blocks}: "
            f"non_bitwise={nonbit} R={r!r} engine R={r_ref!r}")
        assert nonbit == 0 and r == r_ref


def test_noalloc_refuses_bad_arguments():
    hip = Hip()
    d = hip.alloc(64 * 64 * 4)
    try:
        # pitch below the row, a misaligned pitch, the same buffer twice, negative n
        assert pk.pk_sweep_noalloc(pk.PK_F32, 64, 64, 60, d, d + 16384, None, 1) == pk.PK_EINVAL
        assert pk.pk_sweep_noalloc(pk.PK_F32, 3, 3, 5, d, d + 4096, None, 1) == pk.PK_EINVAL
        assert pk.pk_sweep_noalloc(pk.PK_F32, 8, 8, 64, d, d, None, 1) == pk.PK_EINVAL
        assert pk.pk_sweep_noalloc(pk.PK_F32, 8, 8, 64, d, d + 4096, None, -1) == pk.PK_EINVAL
        assert pk.pk_sweep_noalloc(7, 8, 8, 64, d, d + 4096, None, 1) == pk.PK_EINVAL
    finally:
        hip.free(d)

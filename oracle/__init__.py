"""CPU oracle for the 5-point Jacobi and red-black Gauss-Seidel iterations
(test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The HIP engine never imports, links or
calls it, and it imports nothing from the engine.

The arithmetic lives in ``oracle.cpp`` (plain single-threaded C++, built with
``-O2 -ffp-contract=off``); this module only marshals numpy arrays to it. The
header comment of ``oracle.cpp`` cites the passages it follows and lists the
readings taken where the pages are silent.

Pinned by ``tests/test_oracle_pins.py`` (closed forms, invariants, exact
rational brute force); no function here is parity-unpinned.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.cpp")
_LIB = os.path.join(_HERE, "liboracle.so")

_CXXFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c++17", "-Wall", "-Wextra",
             "-shared", "-fPIC"]


def build(force: bool = True) -> str:
    """Compile ``oracle.cpp`` into ``liboracle.so`` next to it (g++)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["g++", *_CXXFLAGS, _SRC, "-o", tmp])
        os.replace(tmp, _LIB)
    return _LIB


class Oracle:
    """ctypes view of one build of ``oracle.cpp`` (the default one, or a test's copy)."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        dp = ctypes.c_void_p
        for name in ("oracle_jacobi_f32", "oracle_jacobi_f64", "oracle_rbgs_f32", "oracle_rbgs_f64"):
            fn = getattr(lib, name)
            fn.restype = ctypes.c_int
            fn.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_double, dp, dp, ctypes.c_int64,
                           dp, ctypes.c_int, dp, dp]
        for name in ("oracle_residual_f32", "oracle_residual_f64"):
            fn = getattr(lib, name)
            fn.restype = ctypes.c_int
            fn.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_double, dp, dp, dp]
        self.lib = lib
        self.path = path

    def jacobi(self, u0: np.ndarray, sweeps: int, f: np.ndarray | None = None,
               h: float | None = None, checkpoints=()):
        """Run ``sweeps`` Jacobi sweeps from ``u0`` (ring held fixed).

        ``u0`` is row-major ``ny x nx`` (row index i = y, column index j = x); its
        outer ring is the Dirichlet data and its interior the initial guess. ``f``
        (same shape and dtype) is the source of -Lap(u) = f; ``None`` means Laplace.
        ``h`` defaults to 1/(nx-1). The residual is recorded before sweep k for each
        k in ``checkpoints`` (non-decreasing, within [0, sweeps]).

        Returns ``(field, residuals)``; ``residuals`` is a float64 array.
        """
        u0, f = _check_field(u0, f)
        ny, nx = u0.shape
        if h is None:
            h = 1.0 / (nx - 1)
        ck = np.ascontiguousarray(np.asarray(checkpoints, dtype=np.int64))
        res = np.zeros(len(ck), dtype=np.float64)
        out = np.empty_like(u0)
        fn = self.lib.oracle_jacobi_f32 if u0.dtype == np.float32 else self.lib.oracle_jacobi_f64
        rc = fn(nx, ny, float(h), _ptr(u0), _ptr(f), int(sweeps), _ptr(ck) if len(ck) else None,
                len(ck), _ptr(out), _ptr(res) if len(ck) else None)
        if rc != 0:
            raise ValueError("oracle rejected its arguments")
        return out, res

    def rbgs(self, u0: np.ndarray, iterations: int, f: np.ndarray | None = None,
             h: float | None = None, checkpoints=()):
        """Run ``iterations`` red-black Gauss-Seidel iterations from ``u0`` in place
        (red = interior nodes with i + j even, updated first; then black). Arguments
        and result as for :meth:`jacobi`, with checkpoints counted in iterations."""
        u0, f = _check_field(u0, f)
        ny, nx = u0.shape
        if h is None:
            h = 1.0 / (nx - 1)
        ck = np.ascontiguousarray(np.asarray(checkpoints, dtype=np.int64))
        res = np.zeros(len(ck), dtype=np.float64)
        out = np.empty_like(u0)
        fn = self.lib.oracle_rbgs_f32 if u0.dtype == np.float32 else self.lib.oracle_rbgs_f64
        rc = fn(nx, ny, float(h), _ptr(u0), _ptr(f), int(iterations), _ptr(ck) if len(ck) else None,
                len(ck), _ptr(out), _ptr(res) if len(ck) else None)
        if rc != 0:
            raise ValueError("oracle rejected its arguments")
        return out, res

    def residual(self, u: np.ndarray, f: np.ndarray | None = None, h: float | None = None) -> float:
        """L2 norm of ``b + (W+E+S+N) - 4u`` over interior cells, in double."""
        u, f = _check_field(u, f)
        ny, nx = u.shape
        if h is None:
            h = 1.0 / (nx - 1)
        r = np.zeros(1, dtype=np.float64)
        fn = self.lib.oracle_residual_f32 if u.dtype == np.float32 else self.lib.oracle_residual_f64
        if fn(nx, ny, float(h), _ptr(u), _ptr(f), _ptr(r)) != 0:
            raise ValueError("oracle rejected its arguments")
        return float(r[0])


def _ptr(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _check_field(u0: np.ndarray, f):
    if u0.ndim != 2 or u0.dtype not in (np.float32, np.float64):
        raise ValueError("u0 must be a 2-D float32 or float64 array")
    u0 = np.ascontiguousarray(u0)
    if f is not None:
        if f.shape != u0.shape:
            raise ValueError("f must have the shape of u0")
        f = np.ascontiguousarray(f, dtype=u0.dtype)
    return u0, f


def compile_copy(src_text: str, out_path: str) -> str:
    """Build a (possibly edited) copy of the oracle source; used by mutation tests."""
    src_path = out_path + ".cpp"
    with open(src_path, "w") as fh:
        fh.write(src_text)
    subprocess.check_call(["g++", *_CXXFLAGS, src_path, "-o", out_path])
    return out_path


def source_text() -> str:
    with open(_SRC) as fh:
        return fh.read()


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        if not os.path.exists(_LIB):
            build(force=False)
        _default = Oracle(_LIB)
    return _default


def jacobi(u0, sweeps, f=None, h=None, checkpoints=()):
    return default().jacobi(u0, sweeps, f=f, h=h, checkpoints=checkpoints)


def rbgs(u0, iterations, f=None, h=None, checkpoints=()):
    return default().rbgs(u0, iterations, f=f, h=h, checkpoints=checkpoints)


def residual(u, f=None, h=None):
    return default().residual(u, f=f, h=h)

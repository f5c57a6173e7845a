"""Seeded synthetic workloads for the Jacobi engine and its oracle.

This module builds inputs only: boundary rings, initial guesses and source
terms, plus the task script each workload runs. It contains none of the
iteration's arithmetic, so both the engine's tests and the oracle can take the
same bytes from it. The random draws come from ``gen.c`` (counter-based
SplitMix64, Box-Muller normals), compiled with gcc into ``_libgen.so``.

Grid convention ("Persistent Kernels: Bridging GPU-CPU Execution", section "The
problem"): N nodes per side including 0 and 1, spacing h = 1/(N-1); row index i
is y = i*h, column index j is x = j*h, arrays are row-major ``ny x nx``. The
"top edge" is row ny-1 (y = 1).
"""

from __future__ import annotations

import ctypes
import dataclasses
import hashlib
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gen.c")
_LIB = os.path.join(_HERE, "_libgen.so")
_CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-Wall", "-Wextra",
           "-shared", "-fPIC"]


def build(force: bool = True) -> str:
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", *_CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        lib.pkgen_uniform.restype = ctypes.c_int
        lib.pkgen_uniform.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int64,
                                      ctypes.c_double, ctypes.c_double, ctypes.c_void_p]
        lib.pkgen_normal.restype = ctypes.c_int
        lib.pkgen_normal.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int64,
                                     ctypes.c_double, ctypes.c_double, ctypes.c_void_p]
        lib.pkgen_sinpi.restype = ctypes.c_int
        lib.pkgen_sinpi.argtypes = [ctypes.c_int64, ctypes.c_double, ctypes.c_double,
                                    ctypes.c_void_p]
        _lib = lib
    return _lib


def uniform(seed: int, stream: int, n: int, lo: float = 0.0, hi: float = 1.0) -> np.ndarray:
    out = np.empty(n, dtype=np.float64)
    if _load().pkgen_uniform(seed, stream, n, lo, hi, ctypes.c_void_p(out.ctypes.data)) != 0:
        raise ValueError("bad uniform draw arguments")
    return out


def normal(seed: int, stream: int, n: int, mean: float = 0.0, sd: float = 1.0) -> np.ndarray:
    out = np.empty(n, dtype=np.float64)
    if _load().pkgen_normal(seed, stream, n, mean, sd, ctypes.c_void_p(out.ctypes.data)) != 0:
        raise ValueError("bad normal draw arguments")
    return out


def sinpi_samples(n: int, h: float, p: float = 1.0) -> np.ndarray:
    """sin(p*pi*j*h) for j = 0..n-1."""
    out = np.empty(n, dtype=np.float64)
    if _load().pkgen_sinpi(n, h, p, ctypes.c_void_p(out.ctypes.data)) != 0:
        raise ValueError("bad sinpi arguments")
    return out


def grid_h(n: int) -> float:
    return 1.0 / (n - 1)


# ---------------------------------------------------------------------------
# Workloads. Each is one of the five configurations the engine is measured on.
# Script steps: ("residual",), ("sweep", n), ("readback",).
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class Workload:
    name: str
    nx: int
    ny: int
    dtype: type
    h: float
    u0: np.ndarray           # ring = Dirichlet data, interior = initial guess
    f: np.ndarray | None     # source of -Lap(u) = f, None for Laplace
    script: list
    description: str

    @property
    def sweeps(self) -> int:
        """Sweeps (Jacobi) plus iterations (red-black) in the script."""
        return sum(s[1] for s in self.script if s[0] in ("sweep", "sweep_rb"))

    @property
    def residual_checkpoints(self) -> list:
        out, k = [], 0
        for s in self.script:
            if s[0] == "sweep":
                k += s[1]
            elif s[0] == "residual":
                out.append(k)
        return out

    @property
    def readback_checkpoints(self) -> list:
        out, k = [], 0
        for s in self.script:
            if s[0] == "sweep":
                k += s[1]
            elif s[0] == "readback":
                out.append(k)
        return out

    @property
    def interior_cells(self) -> int:
        return (self.nx - 2) * (self.ny - 2)

    def digest(self) -> str:
        """SHA-256 over the input bytes (shape, dtype, u0, f)."""
        m = hashlib.sha256()
        m.update(f"{self.nx}x{self.ny}:{np.dtype(self.dtype).name}:{self.h!r}".encode())
        m.update(np.ascontiguousarray(self.u0).tobytes())
        if self.f is not None:
            m.update(np.ascontiguousarray(self.f).tobytes())
        return m.hexdigest()


def _coords(n: int):
    h = grid_h(n)
    return np.arange(n, dtype=np.float64) * h, h


def laplace_harmonic(n: int = 64, sweeps: int = 1000) -> Workload:
    """Laplace, ring u = x^2 - y^2 (discrete harmonic), interior 0, fp32."""
    x, h = _coords(n)
    y = x
    full = (x[None, :] * x[None, :]) - (y[:, None] * y[:, None])
    u0 = np.zeros((n, n), dtype=np.float32)
    u0[0, :] = full[0, :]
    u0[-1, :] = full[-1, :]
    u0[:, 0] = full[:, 0]
    u0[:, -1] = full[:, -1]
    return Workload(f"laplace{n}_harmonic_fp32", n, n, np.float32, h, u0, None,
                    [("sweep", sweeps), ("readback",)],
                    f"{n}x{n} fp32 Laplace, ring x^2-y^2, interior 0, {sweeps} sweeps")


def poisson_uniform(n: int = 256, sweeps: int = 10000, every: int = 100, seed: int = 2) -> Workload:
    """-Lap(u) = f, f ~ U[-1,1] i.i.d. per node, zero ring and interior, fp32."""
    h = grid_h(n)
    f = uniform(seed, 0, n * n, -1.0, 1.0).reshape(n, n).astype(np.float32)
    u0 = np.zeros((n, n), dtype=np.float32)
    script = [("residual",)]
    for _ in range(sweeps // every):
        script += [("sweep", every), ("residual",)]
    script.append(("readback",))
    return Workload(f"poisson{n}_uniform_fp32", n, n, np.float32, h, u0, f, script,
                    f"{n}x{n} fp32 Poisson, f~U[-1,1] seed {seed}, zero ring, {sweeps} sweeps, "
                    f"residual every {every}")


def laplace_random_interior(n: int = 1024, sweeps: int = 5000, every: int = 500,
                            seed: int = 3) -> Workload:
    """Laplace, zero ring, interior ~ U[0,1] i.i.d., fp32."""
    h = grid_h(n)
    u0 = uniform(seed, 0, n * n, 0.0, 1.0).reshape(n, n).astype(np.float32)
    u0[0, :] = 0
    u0[-1, :] = 0
    u0[:, 0] = 0
    u0[:, -1] = 0
    script = [("residual",), ("readback",)]
    for _ in range(sweeps // every):
        script += [("sweep", every), ("residual",), ("readback",)]
    return Workload(f"laplace{n}_random_fp32", n, n, np.float32, h, u0, None, script,
                    f"{n}x{n} fp32 Laplace, interior U[0,1] seed {seed}, zero ring, {sweeps} "
                    f"sweeps, checks every {every}")


def laplace_top_edge(n: int = 4096, sweeps: int = 2000) -> Workload:
    """Laplace, top row (y = 1, corners included) = 1, rest of ring 0, interior 0."""
    h = grid_h(n)
    u0 = np.zeros((n, n), dtype=np.float32)
    u0[-1, :] = 1.0
    return Workload(f"laplace{n}_topedge_fp32", n, n, np.float32, h, u0, None,
                    [("sweep", sweeps), ("readback",)],
                    f"{n}x{n} fp32 Laplace, top edge 1, other edges 0, {sweeps} sweeps")


def poisson_sine_noise(n: int = 8192, sweeps: int = 500, every: int = 50, seed: int = 5,
                       noise_sd: float = 0.01) -> Workload:
    """-Lap(u) = f, f = sin(pi x) sin(pi y) + N(0, sd^2) per node, zero ring, fp64."""
    h = grid_h(n)
    s = sinpi_samples(n, h, 1.0)
    f = s[:, None] * s[None, :]
    f += normal(seed, 2, n * n, 0.0, noise_sd).reshape(n, n)
    u0 = np.zeros((n, n), dtype=np.float64)
    script = [("residual",)]
    for _ in range(sweeps // every):
        script += [("sweep", every), ("residual",)]
    script.append(("readback",))
    return Workload(f"poisson{n}_sine_noise_fp64", n, n, np.float64, h, u0, f, script,
                    f"{n}x{n} fp64 Poisson, f = sin(pi x)sin(pi y) + N(0,{noise_sd}^2) seed "
                    f"{seed}, zero ring, {sweeps} sweeps, residual every {every}")


# The five measured configurations, in the order they are listed for the method.
WORKLOADS = {
    "laplace64": laplace_harmonic,
    "poisson256": poisson_uniform,
    "laplace1024": laplace_random_interior,
    "laplace4096": laplace_top_edge,
    "poisson8192": poisson_sine_noise,
}


def make(name: str, **kw) -> Workload:
    return WORKLOADS[name](**kw)

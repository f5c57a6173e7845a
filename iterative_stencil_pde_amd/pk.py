"""ctypes binding of the engine's C ABI (``include/pk.h``), same names.

Argument marshalling only: every step of the path runs in the HIP library
``_libpk.so``. There is no CPU fallback; loading raises if the library is
missing. Arrays are numpy, row-major ``ny x nx``, float32 or float64.

PyTorch is optional plumbing (a stream handle for ``pk_opts.stream``). Torch
wheels bundle their own HIP runtime; to share one runtime with torch in a
process, import torch before this library is loaded (the library then binds to
the runtime already present, which carries the same soname).
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_libpk.so")

# status codes
PK_OK, PK_EINVAL, PK_ENOMEM, PK_ELAUNCH, PK_EDEVICE, PK_EBUSY, PK_ESTATE, PK_ETIMEDOUT = (
    0, -1, -2, -3, -4, -5, -6, -7)
PK_F32, PK_F64 = 0, 1
PK_PERSISTENT, PK_LAUNCH = 0, 1
PK_LAYOUT_AUTO, PK_LAYOUT_STREAM, PK_LAYOUT_RESIDENT, PK_LAYOUT_REGISTER = 0, 1, 2, 3
PK_SWEEP, PK_RESIDUAL, PK_EXIT, PK_BARRIER, PK_STAMP, PK_SWEEP_RB, PK_SWEEP_UNTIL = 1, 2, 3, 4, 5, 6, 7
PK_BLOCKSYNC = 8
PK_DBG_BROKEN_BARRIER, PK_DBG_TRACE = 0x1, 0x2
PK_TASK_N_MAX = 0x0FFFFFFF
PK_MAX_PASS = 12  # deepest streaming pass (sweeps kept on chip); passes of 1..8 and 12
PK_BARRIER_AUTO, PK_BARRIER_FLAT, PK_BARRIER_TWO_LEVEL, PK_BARRIER_XCD = 0, 1, 2, 3
PK_EXCHANGE_AUTO, PK_EXCHANGE_BARRIER, PK_EXCHANGE_NEIGHBOR, PK_EXCHANGE_TAGGED = 0, 1, 2, 3

EXPORTED = ["pk_opts_default", "pk_create", "pk_submit", "pk_submit_until", "pk_wait", "pk_readback",
            "pk_run_launch_per_iter", "pk_run_graph_per_iter", "pk_get_info", "pk_destroy",
            "pk_strerror", "pk_sweep_noalloc", "pk_trace_read"]
PK_NOALLOC_MAX_BLOCKS = 1024


class pk_opts(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int), ("h", ctypes.c_double), ("mode", ctypes.c_int),
                ("layout", ctypes.c_int), ("threads", ctypes.c_int),
                ("max_blocks", ctypes.c_int), ("halo_depth", ctypes.c_int),
                ("flags", ctypes.c_uint), ("stream", ctypes.c_void_p),
                ("idle_timeout_s", ctypes.c_double), ("barrier", ctypes.c_int),
                ("pass_sweeps", ctypes.c_int), ("band_rows", ctypes.c_int),
                ("exchange", ctypes.c_int), ("reserved", ctypes.c_int * 4)]


class pk_task(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int), ("n", ctypes.c_int)]


class pk_result(ctypes.Structure):
    _fields_ = [("residual", ctypes.c_double), ("sweeps_done", ctypes.c_int64),
                ("device_us", ctypes.c_double), ("errors", ctypes.c_int64),
                ("kind", ctypes.c_int), ("status", ctypes.c_int)]


class pk_info(ctypes.Structure):
    _fields_ = [("nx", ctypes.c_int), ("ny", ctypes.c_int), ("dtype", ctypes.c_int),
                ("mode", ctypes.c_int), ("layout", ctypes.c_int), ("pitch", ctypes.c_int),
                ("grid_blocks", ctypes.c_int), ("threads", ctypes.c_int),
                ("blocks_per_cu_max", ctypes.c_int), ("cus", ctypes.c_int),
                ("halo_depth", ctypes.c_int), ("band_rows", ctypes.c_int),
                ("strips", ctypes.c_int), ("barrier", ctypes.c_int), ("pass_sweeps", ctypes.c_int),
                ("exchange", ctypes.c_int), ("lds_bytes", ctypes.c_size_t),
                ("kernel_ms", ctypes.c_double), ("sweeps_done", ctypes.c_int64),
                ("tasks_done", ctypes.c_int64), ("kernel_launches", ctypes.c_int64),
                ("tasks_carried", ctypes.c_int64), ("wall_clock_khz", ctypes.c_int),
                ("trace_capacity", ctypes.c_int), ("tasks_fused", ctypes.c_int64)]


class PkError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {pk_strerror(status)} ({status})")


_lib = None


def load(path: str = LIB_PATH):
    """Load ``_libpk.so`` (raises if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"engine library not built: {path} (run __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    vp, ip = ctypes.c_void_p, ctypes.c_int
    lib.pk_opts_default.restype = None
    lib.pk_opts_default.argtypes = [ctypes.POINTER(pk_opts)]
    lib.pk_create.restype = ip
    lib.pk_create.argtypes = [ip, ip, vp, vp, ctypes.POINTER(pk_opts), ctypes.POINTER(vp)]
    lib.pk_submit.restype = ip
    lib.pk_submit.argtypes = [vp, pk_task, ctypes.POINTER(ctypes.c_uint64)]
    lib.pk_submit_until.restype = ip
    lib.pk_submit_until.argtypes = [vp, ip, ip, ctypes.c_double, ctypes.POINTER(ctypes.c_uint64)]
    lib.pk_wait.restype = ip
    lib.pk_wait.argtypes = [vp, ctypes.c_uint64, ctypes.c_double, ctypes.POINTER(pk_result)]
    lib.pk_readback.restype = ip
    lib.pk_readback.argtypes = [vp, vp, ctypes.c_size_t]
    lib.pk_run_launch_per_iter.restype = ip
    lib.pk_run_launch_per_iter.argtypes = [vp, ip, ip, ctypes.POINTER(ctypes.c_double)]
    lib.pk_run_graph_per_iter.restype = ip
    lib.pk_run_graph_per_iter.argtypes = [vp, ip, ip, ctypes.POINTER(ctypes.c_double)]
    lib.pk_get_info.restype = ip
    lib.pk_get_info.argtypes = [vp, ctypes.POINTER(pk_info)]
    lib.pk_destroy.restype = ip
    lib.pk_destroy.argtypes = [vp]
    lib.pk_strerror.restype = ctypes.c_char_p
    lib.pk_strerror.argtypes = [ip]
    lib.pk_trace_read.restype = ip
    lib.pk_trace_read.argtypes = [vp, vp, ctypes.c_size_t, ctypes.POINTER(ctypes.c_size_t)]
    lib.pk_sweep_noalloc.restype = ip
    lib.pk_sweep_noalloc.argtypes = [ip, ip, ip, ip, vp, vp, vp, ip, vp, vp]
    _lib = lib
    return lib


def pk_strerror(status: int) -> str:
    try:
        return load().pk_strerror(status).decode()
    except ImportError:
        return f"status {status}"


def _check(rc: int, where: str):
    if rc != PK_OK:
        raise PkError(rc, where)


def pk_opts_default(**kw) -> pk_opts:
    o = pk_opts()
    load().pk_opts_default(ctypes.byref(o))
    for k, v in kw.items():
        if k == "stream" and v is not None and not isinstance(v, int):
            v = int(v)  # e.g. torch.cuda.Stream().cuda_stream
        setattr(o, k, v)
    return o


def pk_create(bc: np.ndarray, src: np.ndarray | None = None, opts: pk_opts | None = None,
              **kw) -> int:
    """Create an engine; returns the opaque handle. ``kw`` fills ``pk_opts``."""
    if bc.ndim != 2 or bc.dtype not in (np.float32, np.float64):
        raise ValueError("bc must be a 2-D float32/float64 array")
    bc = np.ascontiguousarray(bc)
    if opts is None:
        kw.setdefault("dtype", PK_F64 if bc.dtype == np.float64 else PK_F32)
        opts = pk_opts_default(**kw)
    if (opts.dtype == PK_F64) != (bc.dtype == np.float64):
        raise ValueError("bc dtype does not match opts.dtype")
    if src is not None:
        src = np.ascontiguousarray(src, dtype=bc.dtype)
        if src.shape != bc.shape:
            raise ValueError("src must have the shape of bc")
    ny, nx = bc.shape
    h = ctypes.c_void_p()
    rc = load().pk_create(nx, ny, bc.ctypes.data, None if src is None else src.ctypes.data,
                          ctypes.byref(opts), ctypes.byref(h))
    _check(rc, "pk_create")
    return h.value


def pk_submit(eng: int, kind: int, n: int = 0) -> int:
    t = ctypes.c_uint64()
    _check(load().pk_submit(eng, pk_task(kind, n), ctypes.byref(t)), "pk_submit")
    return t.value


def pk_submit_until(eng: int, max_sweeps: int, check_every: int, tol: float) -> int:
    t = ctypes.c_uint64()
    _check(load().pk_submit_until(eng, max_sweeps, check_every, tol, ctypes.byref(t)), "pk_submit_until")
    return t.value


def pk_submit_status(eng: int, kind: int, n: int = 0):
    """Like pk_submit but returns (status, ticket) instead of raising."""
    t = ctypes.c_uint64()
    rc = load().pk_submit(eng, pk_task(kind, n), ctypes.byref(t))
    return rc, t.value


def pk_wait(eng: int, ticket: int, timeout_s: float = 60.0) -> pk_result:
    r = pk_result()
    _check(load().pk_wait(eng, ticket, timeout_s, ctypes.byref(r)), "pk_wait")
    return r


def pk_readback(eng: int, out: np.ndarray) -> np.ndarray:
    if not out.flags.c_contiguous:
        raise ValueError("out must be C-contiguous")
    _check(load().pk_readback(eng, out.ctypes.data, out.nbytes), "pk_readback")
    return out


def pk_run_launch_per_iter(eng: int, n: int, sync_each: bool = False) -> float:
    us = ctypes.c_double()
    _check(load().pk_run_launch_per_iter(eng, n, 1 if sync_each else 0, ctypes.byref(us)),
           "pk_run_launch_per_iter")
    return us.value


def pk_run_graph_per_iter(eng: int, n: int, reps: int) -> float:
    us = ctypes.c_double()
    _check(load().pk_run_graph_per_iter(eng, n, reps, ctypes.byref(us)), "pk_run_graph_per_iter")
    return us.value


def pk_get_info(eng: int) -> pk_info:
    i = pk_info()
    _check(load().pk_get_info(eng, ctypes.byref(i)), "pk_get_info")
    return i


def pk_destroy(eng: int) -> None:
    if eng:
        _check(load().pk_destroy(eng), "pk_destroy")


def pk_sweep_noalloc(dtype: int, nx: int, ny: int, pitch: int, u0: int, u1: int, b: int | None,
                     n: int, residual: int | None = None, stream: int | None = None) -> int:
    """Device pointers as integers (e.g. a torch tensor's data_ptr()); returns the
    status code (0 = queued). Nothing is allocated and nothing synchronizes."""
    return load().pk_sweep_noalloc(dtype, nx, ny, pitch, u0, u1, b, n, residual, stream)


def pk_trace_read(eng: int) -> bytes:
    """The device trace of a PK_DBG_TRACE engine whose kernel has left (raw bytes;
    ``iterative_stencil_pde_amd.trace`` decodes them)."""
    need = ctypes.c_size_t()
    _check(load().pk_trace_read(eng, None, 0, ctypes.byref(need)), "pk_trace_read")
    buf = ctypes.create_string_buffer(need.value)
    _check(load().pk_trace_read(eng, buf, need.value, None), "pk_trace_read")
    return buf.raw


class Engine:
    """Owning wrapper: ``with Engine(bc, f, mode=...) as e: e.sweep(100); ...``."""

    def __init__(self, bc: np.ndarray, src: np.ndarray | None = None, **opts):
        self.shape = bc.shape
        self.dtype = np.dtype(bc.dtype)
        self.h = pk_create(bc, src, **opts)

    def submit(self, kind: int, n: int = 0) -> int:
        return pk_submit(self.h, kind, n)

    def wait(self, ticket: int, timeout_s: float = 60.0) -> pk_result:
        return pk_wait(self.h, ticket, timeout_s)

    def run(self, kind: int, n: int = 0, timeout_s: float = 60.0) -> pk_result:
        return self.wait(self.submit(kind, n), timeout_s)

    def sweep(self, n: int) -> pk_result:
        return self.run(PK_SWEEP, n)

    def sweep_rb(self, n: int) -> pk_result:
        return self.run(PK_SWEEP_RB, n)

    def sweep_until(self, max_sweeps: int, check_every: int, tol: float,
                    timeout_s: float = 60.0) -> pk_result:
        return self.wait(pk_submit_until(self.h, max_sweeps, check_every, tol), timeout_s)

    def residual(self) -> float:
        return self.run(PK_RESIDUAL).residual

    def trace(self) -> bytes:
        return pk_trace_read(self.h)

    def readback(self) -> np.ndarray:
        out = np.empty(self.shape, dtype=self.dtype)
        return pk_readback(self.h, out)

    def info(self) -> pk_info:
        return pk_get_info(self.h)

    def launch_per_iter(self, n: int, sync_each: bool = False) -> float:
        return pk_run_launch_per_iter(self.h, n, sync_each)

    def graph_per_iter(self, n: int, reps: int) -> float:
        return pk_run_graph_per_iter(self.h, n, reps)

    def close(self):
        if self.h:
            h, self.h = self.h, None
            pk_destroy(h)

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

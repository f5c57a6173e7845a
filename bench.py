"""Benchmark: persistent Jacobi engine vs one kernel launch per sweep, one MI355X.

A step is one pass of the workload's whole task script (all its sweeps and
residual checks) on inputs already resident in device memory. Default (the
headline) workload: 8192x8192 fp64 Poisson, f = sin(pi x) sin(pi y) + N(0, 0.01),
500 sweeps with the L2 residual every 50 sweeps (11 residuals).

Prints one JSON line. The persistent kernel is timed from the host (task
submission to completion of the last task of the last step) and, for the
roofline, by HIP events recorded around its single launch on its own stream.
torch.cuda.synchronize() is deliberately not called while the persistent
kernel is resident: a device-wide synchronize would wait for that kernel,
which only leaves on EXIT. Completion of the last task is the device-side
synchronization point instead.

Besides the headline line's required keys it carries: the per-launch baseline
(queued, synchronized after every launch, HIP graph) at the same block count,
the engine's fixed costs, the 4096^2 fp32 workload (`laplace4096`), the three
small workloads with their latency floor (`small_grids`), and the CPU oracle
timed on this host (`cpu_baseline`).
"""

from __future__ import annotations

import argparse
import collections
import copy
import csv
import ctypes
import glob
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from iterative_stencil_pde_amd import inputs, pk  # noqa: E402

PROFILES = os.path.join(ROOT, "profiles")
DEVICE_SOURCES = ["pk_device.h", "pk_persistent.h", "pk_kernels.hip", "pk_kern_stream_f32.hip",
                  "pk_kern_stream_f64.hip", "pk_kern_resident.hip", "pk_kern_register_f32.hip",
                  "pk_kern_register_f64.hip", "pk_shared.h"]
METRIC = ("µs/iteration + Gcell-updates/s (persistent vs per-launch); "
          "HBM GB/s % of peak")
HBM_PEAK_GBS = 8000.0
MALL_BYTES = 256 * 2 ** 20  # Infinity Cache of one MI355X
LAYOUTS = {1: "stream", 2: "resident", 3: "register"}
BARRIERS = {1: "flat", 2: "two_level", 3: "xcd"}
EXCHANGES = {0: None, 1: "barrier", 2: "neighbor", 3: "tagged"}


def say(msg: str):
    """Progress on stderr (stdout carries only the JSON line)."""
    print(msg, file=sys.stderr, flush=True)


class Runtime:
    """The HIP runtime the engine library itself loaded, for plumbing only: a device
    copy of known size (to calibrate byte counters) and releasing the device."""

    def __init__(self):
        pk.load()
        self.rt = ctypes.CDLL("libamdhip64.so.7")
        self.rt.hipMalloc.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_size_t]
        self.rt.hipFree.argtypes = [ctypes.c_void_p]
        self.rt.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]

    def calibration_copy(self, mib: int):
        """One device-to-device copy of mib MiB (the runtime's copy kernel)."""
        n = mib * (1 << 20)
        a, b = ctypes.c_void_p(), ctypes.c_void_p()
        assert self.rt.hipMalloc(ctypes.byref(a), n) == 0 and self.rt.hipMalloc(ctypes.byref(b), n) == 0
        assert self.rt.hipMemcpy(b, a, n, 3) == 0  # hipMemcpyDeviceToDevice
        assert self.rt.hipDeviceSynchronize() == 0
        self.rt.hipFree(a)
        self.rt.hipFree(b)

    def release(self):
        """Free every device resource of this process now, while the process (and
        any profiler attached to it) is still whole, instead of in exit-time
        teardown. Only once no engine is left: a resident persistent kernel would
        make the synchronize wait for it."""
        self.rt.hipDeviceSynchronize()
        self.rt.hipDeviceReset()


# ---- running task scripts ---------------------------------------------------
def step_tasks(w):
    return [s for s in w.script if s[0] in ("sweep", "sweep_rb", "residual")]


def run_steps(e, w, steps: int, timeout_s: float = 600.0):
    """Submit `steps` passes of the script, keeping the task ring full. Returns
    the device time of each step (the sum of its tasks' device times, in us)."""
    pending = collections.deque()
    results = []
    for _ in range(steps):
        for s in step_tasks(w):
            kind = {"sweep": pk.PK_SWEEP, "sweep_rb": pk.PK_SWEEP_RB}.get(s[0], pk.PK_RESIDUAL)
            n = s[1] if s[0] != "residual" else 0
            while True:
                rc, t = pk.pk_submit_status(e.h, kind, n)
                if rc == pk.PK_EBUSY:
                    results.append(e.wait(pending.popleft(), timeout_s))
                    continue
                if rc != pk.PK_OK:
                    raise pk.PkError(rc, "pk_submit")
                pending.append(t)
                break
    while pending:
        results.append(e.wait(pending.popleft(), timeout_s))
    per = len(step_tasks(w))
    return [sum(r.device_us for r in results[i * per:(i + 1) * per]) for i in range(steps)]


def sweep_kind(w):
    return "sweep_rb" if any(s[0] == "sweep_rb" for s in w.script) else "sweep"


def sweeps_only(w):
    """The workload's sweeps as one SWEEP task per step (no residuals)."""
    w1 = copy.copy(w)
    w1.script = [(sweep_kind(w), w.sweeps)]
    return w1


def timed(e, w, steps):
    t0 = time.perf_counter()
    dev = run_steps(e, w, steps)
    return time.perf_counter() - t0, dev


def measure_launch_mode(w, steps, warmup, threads, blocks):
    with pk.Engine(w.u0, w.f, h=w.h, mode=pk.PK_LAUNCH, threads=threads, max_blocks=blocks) as e:
        run_steps(e, w, warmup)
        dt, _ = timed(e, w, steps)
        return dt, e.info()


def launch_graph(w, n, threads, blocks, per_graph=100):
    """HIP-graph form of the per-launch baseline: per_graph sweep launches recorded
    once, replayed until about n sweeps have run (Jacobi only)."""
    per_graph = min(per_graph, n)
    reps = max(1, n // per_graph)
    with pk.Engine(w.u0, w.f, h=w.h, mode=pk.PK_LAUNCH, threads=threads, max_blocks=blocks) as e:
        e.graph_per_iter(per_graph, 1)
        return e.graph_per_iter(per_graph, reps) / (per_graph * reps)


def launch_synced(w, n, threads, blocks):
    """Per-launch baseline with a host synchronization after every launch (red-black:
    after every iteration, i.e. every second launch)."""
    with pk.Engine(w.u0, w.f, h=w.h, mode=pk.PK_LAUNCH, threads=threads, max_blocks=blocks) as e:
        if sweep_kind(w) == "sweep_rb":
            for _ in range(min(n, 50)):
                e.run(pk.PK_SWEEP_RB, 1)
            t0 = time.perf_counter()
            for _ in range(n):
                e.run(pk.PK_SWEEP_RB, 1)
            return (time.perf_counter() - t0) / n * 1e6
        e.launch_per_iter(min(n, 50), True)
        return e.launch_per_iter(n, True) / n


def fixed_costs(e, n_barrier=20000, n_handshake=2000, n_blocksync=100000):
    """Fixed costs of a running persistent engine: a task round trip (SWEEP 0), one
    grid barrier (BARRIER task) and one round of a sub-sweep's block
    synchronization (BLOCKSYNC task), device clock for the last two. The round
    trip is timed as pk_submit + pk_wait called straight from a Python loop with
    their arguments built once (`handshake_us`), and through the Engine wrapper,
    which builds them on every call (`handshake_wrapper_us`)."""
    lib = pk.load()
    task, ticket, res = pk.pk_task(pk.PK_SWEEP, 0), ctypes.c_uint64(), pk.pk_result()
    tref, rref = ctypes.byref(ticket), ctypes.byref(res)
    submit, wait = lib.pk_submit, lib.pk_wait

    def round_trip():
        if submit(e.h, task, tref) != pk.PK_OK or wait(e.h, ticket.value, 60.0, rref) != pk.PK_OK:
            raise RuntimeError("SWEEP 0 round trip failed")

    for _ in range(50):
        round_trip()
    t0 = time.perf_counter()
    for _ in range(n_handshake):
        round_trip()
    handshake_us = (time.perf_counter() - t0) / n_handshake * 1e6
    t0 = time.perf_counter()
    for _ in range(n_handshake):
        e.run(pk.PK_SWEEP, 0)
    wrapper_us = (time.perf_counter() - t0) / n_handshake * 1e6
    e.run(pk.PK_BARRIER, 100)
    barrier_us = e.run(pk.PK_BARRIER, n_barrier).device_us / n_barrier
    e.run(pk.PK_BLOCKSYNC, 1000)
    blocksync_us = e.run(pk.PK_BLOCKSYNC, n_blocksync).device_us / n_blocksync
    return {"handshake_us": round(handshake_us, 3), "handshake_wrapper_us": round(wrapper_us, 3),
            "barrier_us": round(barrier_us, 4),
            "blocksync_us": round(blocksync_us, 5)}


# ---- bytes ------------------------------------------------------------------
def per_unit_bytes(w):
    """Bytes one pass over the field must move (every interior cell's u read and
    written once, b read once when present) and one residual (u and b read)."""
    es = np.dtype(w.dtype).itemsize
    has_b = w.f is not None
    return (w.interior_cells * es * (2 + (1 if has_b else 0)),
            w.interior_cells * es * (1 + (1 if has_b else 0)))


SHALLOW_PASS = 8  # the deepest pass that also sums the residual, and red-black passes


def pass_depths(n, depth, rb=False):
    """The passes a streaming task of n sweeps (red-black: half-sweeps) runs at the
    engine's depth, as the kernel splits it: depth-deep passes, a depth it does not
    carry (9..11) as 8, and a last Jacobi pass of at most 8 (it also sums the
    residual: a 12-sweep tail runs as 4 + 8)."""
    out = []
    while n > 0:
        k = min(depth, n)
        if k > SHALLOW_PASS and (rb or k != pk.PK_MAX_PASS):
            k = SHALLOW_PASS
        if k == n and k > SHALLOW_PASS:
            k = n - SHALLOW_PASS
        out.append(k)
        n -= k
    return out


def default_depth(w):
    """The planner's pass depth: 12 where the streamed arrays (u, u', b) exceed the
    256 MiB Infinity Cache, else 8."""
    es = np.dtype(w.dtype).itemsize
    pitch_bytes = -(-w.nx * es // 256) * 256
    streamed = pitch_bytes * w.ny * (3 if w.f is not None else 2)
    return pk.PK_MAX_PASS if streamed > MALL_BYTES else SHALLOW_PASS


def fuses(w, pass_sweeps):
    """Whether a persistent streaming engine runs a SWEEP task's last pass on into
    the next SWEEP task (a RESIDUAL between them summed inside that pass): the fp64
    kernels at depth 12, where the tasks are queued ahead (the bench keeps the ring
    full)."""
    return np.dtype(w.dtype) == np.float64 and pass_sweeps == pk.PK_MAX_PASS


def script_counts(w, pass_sweeps, fuse=None, stats=None):
    """(sweeps, passes, residual reads) of one step of a persistent streaming
    engine, as the kernel plans it: each SWEEP task runs the passes of pass_depths
    (k = 1: one pass per sweep); a RESIDUAL right after a Jacobi SWEEP task of
    n > 0 sweeps reads nothing (its partials were summed by that task's last pass),
    any other reads u and b. With fusion (fuses()): a SWEEP task with more than P
    sweeps left runs P-deep passes, and where its last t <= P sweeps are followed
    by a RESIDUAL and a SWEEP of at least P - t sweeps (t = P: at least P), they
    run as one P-deep pass that also applies the first P - t sweeps of the later
    task and sums the RESIDUAL on the way (t = P: a pass of their own, then the
    later task's first P sweeps with the residual of level 0). A RESIDUAL of a
    field no pass has summed, followed by a SWEEP of at least P, runs that task's
    first pass and sums its level 0 instead of reading the field. `stats` (a dict),
    if given, receives the number of such fused tasks ("fused")."""
    if fuse is None:
        fuse = fuses(w, pass_sweeps)
    tasks = step_tasks(w)
    P = max(1, pass_sweeps)
    sweeps = passes = residuals = fused_tails = 0
    ready = False  # the last pass summed the residual of the field as it is now
    pre = 0        # sweeps of the next SWEEP task already applied
    for idx, t in enumerate(tasks):
        if t[0] == "residual":
            nxt = tasks[idx + 1:idx + 2]
            if not ready and fuse and P == pk.PK_MAX_PASS and nxt and nxt[0][0] == "sweep" and nxt[0][1] >= P:
                # the next SWEEP task's first pass runs here and sums level 0
                passes += 1
                pre = P
                fused_tails += 1
            else:
                residuals += 0 if ready else 1
            ready = False
            continue
        rb = t[0] == "sweep_rb"
        sweeps += t[1]
        n = t[1] * (2 if rb else 1)  # red-black: two half-sweeps
        if not rb:
            n -= pre
        pre = 0
        fz = fuse and not rb and P == pk.PK_MAX_PASS
        s, fused, ran = 0, False, False
        while s < n:
            left = n - s
            k = P if fz and left > P else pass_depths(left, P, rb)[0]
            passes += 1
            ran = True
            res = s + k >= n and not rb and P > 1
            ready = res
            s += k
            rest = n - s
            if fz and 0 < rest <= P:
                nxt = tasks[idx + 1:idx + 3]
                fused = len(nxt) == 2 and nxt[0][0] == "residual" and nxt[1][0] == "sweep" \
                    and nxt[1][1] >= (P - rest if rest < P else P)
                if fused:
                    break
        if fused:
            t = n - s
            if t == P:  # a pass of its own, then the later task's first P sweeps tap level 0
                passes += 1
                t = 0
            passes += 1
            pre = P - t
            fused_tails += 1
            ready = True
        if rb and ran:
            ready = False
    if stats is not None:
        stats["fused"] = fused_tails
    return sweeps, passes, residuals


def algorithmic_bytes(w, pass_sweeps):
    """(per-sweep bytes of the method, bytes of one step counted per pass)."""
    per_pass, per_res = per_unit_bytes(w)
    _, passes, residuals = script_counts(w, pass_sweeps)
    return per_pass, passes * per_pass + residuals * per_res


# ---- stored HBM counter traffic (rocprofv3 --pmc runs) ----------------------
def device_source_sha() -> str:
    """Hash of the device code: stored counter traffic is valid for this hash only."""
    h = hashlib.sha256()
    for name in DEVICE_SOURCES:
        with open(os.path.join(ROOT, "iterative_stencil_pde_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_file(workload: str) -> str:
    return os.path.join(PROFILES, f"pk_persistent_{workload}_traffic.json")


def stored_traffic(workload: str, launch_algorithmic_bytes: float):
    """Counter bytes (FETCH_SIZE + WRITE_SIZE, calibrated on a copy of known size)
    for a launch of this many algorithmic bytes: the stored ratio of counter to
    algorithmic bytes times this launch's algorithmic bytes. None when absent or
    taken on other device code."""
    path = traffic_file(workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("device_source_sha") != device_source_sha():
        return None
    return rec["bytes_per_launch"] / rec["algorithmic_bytes_per_launch"] * launch_algorithmic_bytes


def _counter_rows(d):
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    with open(files[0]) as f:
        return list(csv.DictReader(f))


def fold_traffic(fetch_dir, write_dir, workload, launch_algorithmic_bytes, copy_mib):
    """Turn two counter runs (each: a copy of copy_mib MiB, then the headline
    launch) into the stored traffic record."""
    def per_kernel(d, counter):
        out = collections.defaultdict(list)
        rows = sorted(_counter_rows(d), key=lambda r: int(r.get("Dispatch_Id", 0) or 0))
        for r in rows:
            if r["Counter_Name"] == counter:
                out[r["Kernel_Name"]].append(float(r["Counter_Value"]))
        return out
    fetch = per_kernel(fetch_dir, "FETCH_SIZE")
    write = per_kernel(write_dir, "WRITE_SIZE")
    copy_bytes = copy_mib * (1 << 20)

    def one(table, pattern, what):
        keys = [k for k in table if pattern in k and "Rect" not in k]
        if not keys or not table[keys[0]]:
            raise SystemExit(f"no {what} dispatch ({pattern}) in the counters")
        return table[keys[0]][0]  # the first dispatch: the calibration copy / the headline launch

    copy_key = "copyBuffer"  # the runtime's device-to-device copy kernel
    f_scale = copy_bytes / (one(fetch, copy_key, "copy") * 1024.0)
    w_scale = copy_bytes / (one(write, copy_key, "copy") * 1024.0)
    f_kib = one(fetch, "pk_persistent", "persistent")
    w_kib = one(write, "pk_persistent", "persistent")
    total = f_kib * 1024.0 * f_scale + w_kib * 1024.0 * w_scale
    rec = {"workload": workload, "device_source_sha": device_source_sha(),
           "fetch_kib": f_kib, "write_kib": w_kib, "fetch_scale": round(f_scale, 4),
           "write_scale": round(w_scale, 4), "bytes_per_launch": total,
           "algorithmic_bytes_per_launch": launch_algorithmic_bytes,
           "ratio_to_algorithmic": total / launch_algorithmic_bytes,
           "note": "FETCH_SIZE and WRITE_SIZE of the first pk_persistent dispatch, each scaled by "
                   "known bytes / counter of a device copy of the same run; Infinity Cache hits count"}
    with open(traffic_file(workload), "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


# ---- the persistent engine on one workload ------------------------------------
def persistent_run(w, steps, warmup, opts, pure=True):
    """One engine, one launch: warmup + timed steps of the script, then (pure) the
    same number of pure-SWEEP steps. Returns timings, plan and the launch's
    kernel time (HIP events around the launch on its stream)."""
    with pk.Engine(w.u0, w.f, h=w.h, mode=pk.PK_PERSISTENT, **opts) as e:
        info = e.info()
        run_steps(e, w, warmup)
        dt, dev = timed(e, w, steps)
        pure_dt = None
        if pure:
            dt_p, _ = timed(e, sweeps_only(w), steps)
            pure_dt = dt_p
        e.wait(e.submit(pk.PK_EXIT))
        end = e.info()
    return {"dt": dt, "dev": sorted(dev), "pure_dt": pure_dt, "info": info, "end": end}


def roofline_stream(w, r, steps, warmup, traffic_key):
    """HBM roofline of a persistent streaming launch. The unit is one pass over the
    field (up to k sweeps kept on chip): its algorithmic bytes read u and b once and
    write u once; a residual that the pass before it did not sum reads u and b. The
    counter bytes (stored, same device code)
    add what the kernel really moves (halo rows, overlap lanes, polling words; Infinity
    Cache hits count)."""
    info, end = r["info"], r["end"]
    k = info.pass_sweeps
    per_sweep, step_pass = algorithmic_bytes(w, k)
    pure_pass = algorithmic_bytes(sweeps_only(w), k)[1]
    n_script = steps + warmup
    model = {}
    script_counts(w, k, stats=model)
    launch_alg = n_script * step_pass + (steps * pure_pass if r["pure_dt"] is not None else 0)
    launch_sweeps = w.sweeps * (n_script + (steps if r["pure_dt"] is not None else 0))
    kernel_s = end.kernel_ms / 1e3
    achieved = launch_alg / kernel_s / 1e9
    traffic = stored_traffic(traffic_key, launch_alg)
    working_set = (3 if w.f is not None else 2) * w.ny * info.pitch * np.dtype(w.dtype).itemsize
    out = {
        "bound": "hbm",
        "achieved": round(achieved, 2),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4),
        "traffic": traffic,
        "kernel": "pk_persistent (streaming passes)",
        "kernel_ms": round(end.kernel_ms, 3),
        "launches": 1,
        "pass_sweeps": k,
        "algorithmic_unit": "one pass of up to k sweeps: u read and written once, b read once; a residual "
                            "not summed by the pass before it reads u and b",
        "algorithmic_bytes_per_launch": launch_alg,
        # SWEEP tasks whose tail ran on into the next SWEEP task: the pass count above
        # assumes the model's number, the device reports how many it fused
        "fused_tails": {"model": model["fused"] * n_script, "device": int(end.tasks_fused)},
        "counter_GBps": round(traffic / kernel_s / 1e9, 2) if traffic else None,
        "counter_frac": round(traffic / kernel_s / 1e9 / HBM_PEAK_GBS, 4) if traffic else None,
        "counter_to_algorithmic": round(traffic / launch_alg, 4) if traffic else None,
        # the same launch counted as if every sweep streamed the field (the pages'
        # "effective bandwidth"); above the peak because passes keep k sweeps on chip
        "sweep_equivalent_GBps": round(per_sweep * launch_sweeps / kernel_s / 1e9, 1),
        "regime": ("HBM: the working set (%.0f MiB) exceeds the 256 MiB Infinity Cache" % (working_set / 2 ** 20)
                   if working_set > MALL_BYTES else
                   "Infinity Cache: the working set (%.0f MiB) fits the 256 MiB Infinity Cache, so counter "
                   "bytes are mostly cache hits, not HBM traffic" % (working_set / 2 ** 20)),
    }
    return out


def plan_dict(info):
    return {"layout": LAYOUTS[info.layout], "grid_blocks": info.grid_blocks, "threads": info.threads,
            "halo_depth": info.halo_depth, "band_rows": info.band_rows,
            "barrier": BARRIERS[info.barrier], "exchange": EXCHANGES[info.exchange],
            "pass_sweeps": info.pass_sweeps}


def small_grid(name, steps=2, warmup=1):
    """A small workload: persistent (script and pure sweeps) against launches, with the
    latency floor of its tile plan. These grids live on chip: the bound is the
    synchronization per sub-sweep, not HBM."""
    w = inputs.make(name)
    say(f"[bench] small grid {name}")
    r = persistent_run(w, steps, warmup, {})
    with pk.Engine(w.u0, w.f, h=w.h) as e:
        costs = fixed_costs(e, n_barrier=5000, n_handshake=500, n_blocksync=50000)
    info = r["info"]
    us_script = r["dt"] / (w.sweeps * steps) * 1e6
    us_pure = r["pure_dt"] / (w.sweeps * steps) * 1e6
    ldt, _ = measure_launch_mode(w, steps, 1, info.threads, info.grid_blocks)
    us_launch = ldt / (w.sweeps * steps) * 1e6
    us_graph = launch_graph(w, min(w.sweeps, 2000), info.threads, info.grid_blocks)
    us_synced = launch_synced(w, min(w.sweeps, 500), info.threads, info.grid_blocks)
    m = info.halo_depth if info.grid_blocks > 1 else 0
    # every tile sweep is one sub-sweep per block, each with one block
    # synchronization; every m sweeps the blocks also exchange halo rows, which
    # costs at least one device round trip (the grid barrier's share is given)
    floor = costs["blocksync_us"]
    return {
        "workload": w.name,
        "plan": plan_dict(info),
        "us_per_iteration": round(us_script, 4),
        "us_per_iteration_sweep_task": round(us_pure, 4),
        "per_launch_us_per_iteration": {"queued": round(us_launch, 4), "synced": round(us_synced, 4),
                                        "graph": round(us_graph, 4)},
        "speedup_vs_queued": round(us_launch / us_script, 3),
        "speedup_vs_graph": round(us_graph / us_script, 3),
        "overheads": costs,
        "roofline": {
            "bound": "latency",
            "floor_us_per_sweep": round(floor, 4),
            "floor": "one block synchronization (LDS write, block barrier, LDS read) per sub-sweep, "
                     "measured by the BLOCKSYNC task; a sweep of a tile plan is one sub-sweep",
            "grid_barrier_share_us_per_sweep": round(costs["barrier_us"] / m, 4) if m else 0.0,
            "frac": round(floor / us_pure, 4),
        },
    }


def laplace4096_entry(steps=3, warmup=1):
    w = inputs.make("laplace4096")
    say("[bench] laplace4096")
    r = persistent_run(w, steps, warmup, {})
    info = r["info"]
    us = r["dt"] / (w.sweeps * steps) * 1e6
    ldt, _ = measure_launch_mode(w, 1, 1, info.threads, info.grid_blocks)
    us_launch = ldt / w.sweeps * 1e6
    return {
        "workload": w.name,
        "plan": plan_dict(info),
        "us_per_iteration": round(us, 4),
        "value": round(w.interior_cells * w.sweeps * steps / r["dt"] / 1e9, 3),
        "unit": "Gcell-updates/s",
        "per_launch_us_per_iteration": round(us_launch, 4),
        "speedup_vs_queued": round(us_launch / us, 3),
        "roofline": roofline_stream(w, r, steps, warmup, "laplace4096"),
    }


# ---- the CPU oracle on this host ---------------------------------------------
def host_cpu():
    model = platform.processor() or ""
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count()
    return model, os.cpu_count(), avail


def cpu_baseline(w, blocks=None):
    """The single-threaded C++ oracle, as it stands, on this host, on the first
    `blocks` blocks of the script (a residual, then `blocks` times sweeps and a
    residual); None runs the whole script."""
    import oracle
    res_ck = w.residual_checkpoints
    every = res_ck[1] - res_ck[0] if len(res_ck) > 1 else w.sweeps
    sweeps = w.sweeps if blocks is None else min(w.sweeps, blocks * every)
    ck = [c for c in res_ck if c <= sweeps]
    say(f"[bench] cpu oracle: {sweeps} sweeps, {len(ck)} residuals")
    t0 = time.perf_counter()
    oracle.jacobi(w.u0, sweeps, f=w.f, h=w.h, checkpoints=ck)
    dt = time.perf_counter() - t0
    model, ncpu, avail = host_cpu()
    return {"value": round(w.interior_cells * sweeps / dt / 1e9, 4), "unit": "Gcell-updates/s",
            "cores": 1, "kind": "oracle",
            "us_per_iteration": round(dt / sweeps * 1e6, 1),
            "sample": f"{'the whole' if blocks is None else 'the first %d blocks of the' % blocks} "
                      f"{w.name} script ({sweeps} sweeps, {len(ck)} residuals), single-threaded C++ "
                      f"oracle, {dt:.1f} s",
            "host": {"cpu_model": model, "nproc": ncpu, "cpus_available": avail}}


# ---- main -----------------------------------------------------------------------
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="poisson8192", choices=sorted(inputs.WORKLOADS))
    ap.add_argument("--layout", default="auto", choices=["auto", "stream", "resident", "register"])
    ap.add_argument("--threads", type=int, default=0)
    ap.add_argument("--max-blocks", type=int, default=0)
    ap.add_argument("--halo", type=int, default=0)
    ap.add_argument("--barrier", default="auto", choices=["auto", "flat", "two_level", "xcd"])
    ap.add_argument("--exchange", default="auto", choices=["auto", "barrier", "neighbor", "tagged"],
                    help="tile layouts: halo exchange by grid barrier, neighbour flags or tagged words; "
                         "streaming passes: grid barrier or neighbour counters per XCD")
    ap.add_argument("--pass-sweeps", type=int, default=0, help="stream layout: sweeps per pass")
    ap.add_argument("--band-rows", type=int, default=0, help="stream passes: rows per band")
    ap.add_argument("--launch-steps", type=int, default=0,
                    help="steps for the per-launch comparison (default: same as --steps)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-full", action="store_true",
                    help="time the oracle on the whole script instead of its first two blocks")
    ap.add_argument("--no-extra", action="store_true",
                    help="leave out the 4096^2 and small-grid entries")
    ap.add_argument("--method", default="jacobi", choices=["jacobi", "rb"],
                    help="rb: the same script with red-black Gauss-Seidel iterations instead of "
                         "Jacobi sweeps (one iteration = red then black half-sweep)")
    ap.add_argument("--idle-timeout", type=float, default=0.0,
                    help="persistent kernel idle timeout in seconds (0 = engine default)")
    ap.add_argument("--main-only", action="store_true",
                    help="only the headline persistent launch (for counter collection)")
    ap.add_argument("--fold-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="store the traffic of two rocprofv3 counter runs of this workload "
                         "(made with --main-only --calibrate-copy MIB) and exit")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="first run a device-to-device copy of MIB MiB (a plain copy kernel "
                         "of known size, to scale HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(json.dumps({"error": "this engine runs on one GPU; --gpus must be 1 "
                          "(the multi-GPU row-band design is described, not built)"}))
        sys.exit(2)

    w = inputs.make(args.workload)
    if args.method == "rb":
        w.script = [("sweep_rb", s[1]) if s[0] == "sweep" else s for s in w.script]
    layout = {"auto": pk.PK_LAYOUT_AUTO, "stream": pk.PK_LAYOUT_STREAM,
              "resident": pk.PK_LAYOUT_RESIDENT, "register": pk.PK_LAYOUT_REGISTER}[args.layout]
    barrier = {"auto": pk.PK_BARRIER_AUTO, "flat": pk.PK_BARRIER_FLAT,
               "two_level": pk.PK_BARRIER_TWO_LEVEL, "xcd": pk.PK_BARRIER_XCD}[args.barrier]
    exchange = {"auto": pk.PK_EXCHANGE_AUTO, "barrier": pk.PK_EXCHANGE_BARRIER,
                "neighbor": pk.PK_EXCHANGE_NEIGHBOR, "tagged": pk.PK_EXCHANGE_TAGGED}[args.exchange]
    opts = dict(layout=layout, threads=args.threads, max_blocks=args.max_blocks,
                halo_depth=args.halo, idle_timeout_s=args.idle_timeout, barrier=barrier,
                pass_sweeps=args.pass_sweeps, band_rows=args.band_rows, exchange=exchange)
    traffic_key = w.name.split("_")[0]

    if args.fold_traffic:
        # the launch of a --main-only run of a streaming workload: its algorithmic
        # bytes with the passes it ran (the planner's default depth unless given)
        k = args.pass_sweeps or default_depth(w)
        per_step = algorithmic_bytes(w, k)[1]
        pure = algorithmic_bytes(sweeps_only(w), k)[1]
        fold_traffic(args.fold_traffic[0], args.fold_traffic[1], traffic_key,
                     (args.steps + args.warmup) * per_step + args.steps * pure, args.calibrate_copy or 1024)
        return

    rt = Runtime()
    try:
        run(args, w, opts, traffic_key, rt)
    finally:
        rt.release()


def run(args, w, opts, traffic_key, rt):
    if args.calibrate_copy:
        rt.calibration_copy(args.calibrate_copy)

    cells_per_step = w.interior_cells * w.sweeps
    say(f"[bench] {w.name}: persistent, {args.warmup} + {args.steps} steps")
    r = persistent_run(w, args.steps, args.warmup, opts)
    info, end = r["info"], r["end"]
    stream = info.layout == pk.PK_LAYOUT_STREAM
    if args.main_only:
        print(json.dumps({"workload": w.name, "kernel_ms": end.kernel_ms,
                          "us_per_iteration": round(r["dt"] / (w.sweeps * args.steps) * 1e6, 4)}), flush=True)
        return
    value = cells_per_step * args.steps / r["dt"] / 1e9
    us_iter = r["dt"] / (w.sweeps * args.steps) * 1e6
    us_pure = r["pure_dt"] / (w.sweeps * args.steps) * 1e6

    # fixed costs, on an engine of another kernel instance with the same plan (the
    # headline kernel's only launch is the timed one): the same grid without b
    say("[bench] fixed costs")
    w_fixed = copy.copy(w)
    w_fixed.f = None
    t0 = time.perf_counter()
    with pk.Engine(w_fixed.u0, None, h=w.h, **opts) as e:
        create_ms = (time.perf_counter() - t0) * 1e3
        fixed = dict(create_launch_ms=round(create_ms, 3), **fixed_costs(e))
        fixed["plan_grid_blocks"] = e.info().grid_blocks

    # per-launch baseline, same block count as the persistent grid
    say("[bench] per-launch baseline")
    lsteps = args.launch_steps or args.steps
    ldt, linfo = measure_launch_mode(w, lsteps, 1, info.threads, info.grid_blocks)
    lvalue = cells_per_step * lsteps / ldt / 1e9
    lsync = launch_synced(w, min(w.sweeps, 2000), info.threads, info.grid_blocks)
    lgraph = launch_graph(w, min(w.sweeps, 10000), info.threads, info.grid_blocks) \
        if sweep_kind(w) == "sweep" else None

    n_res = sum(1 for s in step_tasks(w) if s[0] == "residual")
    if stream:
        roof = roofline_stream(w, r, args.steps, args.warmup, traffic_key)
    else:
        roof = {"bound": "latency", "achieved": None, "peak": None, "unit": "us", "frac": None,
                "traffic": None, "kernel_ms": round(end.kernel_ms, 3),
                "note": "tile layouts keep the field on chip; see small_grids for their latency floor"}
    rec = {
        "metric": METRIC,
        "value": round(value, 4),
        "unit": "Gcell-updates/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["dt"] / args.steps * 1e3, 4),
        # each timed step's time on the device clock (its tasks' device times summed)
        "ms_per_step_device": {"min": round(r["dev"][0] / 1e3, 4),
                               "median": round(r["dev"][len(r["dev"]) // 2] / 1e3, 4)},
        "us_per_iteration": round(us_iter, 4),
        "us_per_iteration_sweep_task": round(us_pure, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f64" if w.dtype == np.float64 else "f32",
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "method": "red_black_gauss_seidel" if args.method == "rb" else "jacobi",
            "shape": [w.ny, w.nx],
            "sweeps_per_step": w.sweeps,
            "residuals_per_step": n_res,
            "mode": "persistent",
            **plan_dict(info),
        },
        "per_launch": {
            "value": round(lvalue, 4),
            "us_per_iteration": round(ldt / (w.sweeps * lsteps) * 1e6, 4),
            "us_per_iteration_synced": round(lsync, 4),
            "us_per_iteration_graph": round(lgraph, 4) if lgraph else None,
            "steps": lsteps,
            "grid_blocks": linfo.grid_blocks,
            "kernel_launches_per_step": (2 if args.method == "rb" else 1) * w.sweeps + 2 * n_res,
            "speedup_persistent": round(value / lvalue, 3),
            "speedup_persistent_vs_graph": round(lgraph / us_iter, 3) if lgraph else None,
        },
        "overheads": dict(fixed, tasks_carried=int(end.tasks_carried), tasks_done=int(end.tasks_done),
                          tasks_fused=int(end.tasks_fused)),
        "roofline": roof,
    }
    if not args.no_extra and args.workload == "poisson8192" and args.method == "jacobi":
        rec["laplace4096"] = laplace4096_entry()
        rec["small_grids"] = [small_grid(n) for n in ("laplace64", "poisson256", "laplace1024")]
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w, None if args.cpu_full else 2)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()

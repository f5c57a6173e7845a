"""Benchmark: persistent Jacobi engine vs one kernel launch per sweep, one MI355X.

A step is one pass of the workload's whole task script (all its sweeps and
residual checks) on inputs already resident in device memory. Default workload:
256x256 fp32 Poisson, 10,000 sweeps with an L2 residual every 100 sweeps.

Prints one JSON line. The persistent kernel is timed from the host (task
submission to completion of the last task of the last step) and, for the
roofline, by HIP events recorded around its single launch on its own stream.
torch.cuda.synchronize() is deliberately not called while the persistent
kernel is resident: a device-wide synchronize would wait for that kernel,
which only leaves on EXIT. Completion of the last task is the device-side
synchronization point instead.
"""

from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from iterative_stencil_pde_amd import inputs, pk  # noqa: E402

PROFILES = os.path.join(ROOT, "profiles")
DEVICE_SOURCES = ["pk_device.h", "pk_kernels.hip", "pk_shared.h"]
METRIC = ("µs/iteration + Gcell-updates/s (persistent vs per-launch); "
          "HBM GB/s % of peak")
HBM_PEAK_GBS = 8000.0


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


def algorithmic_bytes(w):
    """Minimum bytes a step must move: every interior cell read and written once
    per sweep (plus b read once when present); each residual reads u (and b)."""
    es = np.dtype(w.dtype).itemsize
    has_b = w.f is not None
    per_sweep = w.interior_cells * es * (2 + (1 if has_b else 0))
    per_residual = w.interior_cells * es * (1 + (1 if has_b else 0))
    n_res = sum(1 for s in step_tasks(w) if s[0] == "residual")
    return w.sweeps * per_sweep + n_res * per_residual, per_sweep


def measure(w, steps, warmup, **opts):
    with pk.Engine(w.u0, w.f, h=w.h, **opts) as e:
        info0 = e.info()
        run_steps(e, w, warmup)
        t0 = time.perf_counter()
        step_us = run_steps(e, w, steps)
        t1 = time.perf_counter()
        if opts.get("mode", pk.PK_PERSISTENT) == pk.PK_PERSISTENT:
            e.wait(e.submit(pk.PK_EXIT))
        info1 = e.info()
    measure.step_us = step_us  # device time per timed step (persistent mode)
    return t1 - t0, info0, info1


def sweep_kind(w):
    return "sweep_rb" if any(s[0] == "sweep_rb" for s in w.script) else "sweep"


def sweep_only(w, steps, warmup, **opts):
    """Variant (i): the same sweeps as one SWEEP task per step, no residuals."""
    import copy
    w1 = copy.copy(w)
    w1.script = [(sweep_kind(w), w.sweeps)]
    dt, _, _ = measure(w1, steps, warmup, **opts)
    return dt / (w.sweeps * steps) * 1e6


def overheads(w, opts, n_barrier=20000, n_handshake=2000):
    """Fixed costs of the persistent engine with the same plan: create + launch,
    one task round trip (SWEEP 0), and one grid barrier (a BARRIER task)."""
    t0 = time.perf_counter()
    e = pk.Engine(w.u0, w.f, h=w.h, mode=pk.PK_PERSISTENT, **opts)
    create_ms = (time.perf_counter() - t0) * 1e3
    with e:
        for _ in range(50):
            e.run(pk.PK_SWEEP, 0)
        t0 = time.perf_counter()
        for _ in range(n_handshake):
            e.run(pk.PK_SWEEP, 0)
        handshake_us = (time.perf_counter() - t0) / n_handshake * 1e6
        e.run(pk.PK_BARRIER, 100)
        r = e.run(pk.PK_BARRIER, n_barrier)
        barrier_us = r.device_us / n_barrier
    return {"create_launch_ms": round(create_ms, 3), "handshake_us": round(handshake_us, 3),
            "barrier_us": round(barrier_us, 4)}


def launch_graph(w, n, threads, blocks, per_graph=100):
    """HIP-graph form of the per-launch baseline: per_graph sweep launches recorded
    once, replayed until about n sweeps have run (Jacobi only)."""
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


def device_source_sha() -> str:
    """Hash of the device code: stored counter traffic is valid for this hash only."""
    h = hashlib.sha256()
    for name in DEVICE_SOURCES:
        with open(os.path.join(ROOT, "iterative_stencil_pde_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_file(workload: str) -> str:
    return os.path.join(PROFILES, f"pk_persistent_{workload}_traffic.json")


def stored_traffic(workload: str, steps_in_launch: int):
    """HBM-side bytes of one persistent launch from stored rocprofv3 counters
    (FETCH_SIZE and WRITE_SIZE, calibrated on a copy of known size), scaled to
    this launch's step count; None when absent or taken on other device code."""
    path = traffic_file(workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("device_source_sha") != device_source_sha():
        return None
    return rec["bytes_per_step"] * steps_in_launch


def default_plan(args) -> bool:
    """True when the run uses the plan and method the stored counters were taken
    with (Jacobi, every planner choice left to the planner)."""
    return (args.method == "jacobi" and args.layout == "auto" and not args.threads and not args.max_blocks
            and not args.halo and args.barrier == "auto" and args.exchange == "auto" and not args.pass_sweeps
            and not args.band_rows)


def _counter_rows(d):
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    with open(files[0]) as f:
        return list(csv.DictReader(f))


def fold_traffic(fetch_dir, write_dir, workload, steps_in_launch, copy_mib):
    """Turn two counter runs (each: a copy of copy_mib MiB, then the persistent
    launch of steps_in_launch steps) into the stored traffic record."""
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
        return table[keys[0]][0]  # the first dispatch: the calibration copy / the timed launch

    copy_key = "copyBuffer"  # the runtime's device-to-device copy kernel
    f_scale = copy_bytes / (one(fetch, copy_key, "copy") * 1024.0)
    w_scale = copy_bytes / (one(write, copy_key, "copy") * 1024.0)
    f_kib = one(fetch, "pk_persistent", "persistent")
    w_kib = one(write, "pk_persistent", "persistent")
    total = f_kib * 1024.0 * f_scale + w_kib * 1024.0 * w_scale
    rec = {"workload": workload, "device_source_sha": device_source_sha(),
           "steps_in_profiled_launch": steps_in_launch,
           "fetch_kib": f_kib, "write_kib": w_kib, "fetch_scale": round(f_scale, 4),
           "write_scale": round(w_scale, 4), "bytes_per_launch": total,
           "bytes_per_step": total / steps_in_launch,
           "note": "FETCH_SIZE and WRITE_SIZE of the first pk_persistent dispatch, each scaled by "
                   "known bytes / counter of a device copy of the same run; MALL hits count"}
    with open(traffic_file(workload), "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


def cpu_baseline(w, budget_s: float = 10.0):
    import oracle
    ck = w.residual_checkpoints
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.jacobi(w.u0, w.sweeps, f=w.f, h=w.h, checkpoints=ck)
        reps += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    cells = w.interior_cells * w.sweeps * reps
    return {"value": round(cells / dt / 1e9, 4), "unit": "Gcell-updates/s", "cores": 1,
            "kind": "oracle",
            "sample": f"{reps} full run(s) of the {w.name} script ({w.sweeps} sweeps, "
                      f"{len(ck)} residuals), single-threaded C++ oracle, {dt:.1f}s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="poisson256", choices=sorted(inputs.WORKLOADS))
    ap.add_argument("--layout", default="auto", choices=["auto", "stream", "resident", "register"])
    ap.add_argument("--threads", type=int, default=0)
    ap.add_argument("--max-blocks", type=int, default=0)
    ap.add_argument("--halo", type=int, default=0)
    ap.add_argument("--barrier", default="auto", choices=["auto", "flat", "two_level", "xcd"])
    ap.add_argument("--exchange", default="auto", choices=["auto", "barrier", "neighbor", "tagged"],
                    help="tile layouts: halo exchange by grid barrier, neighbour flags or tagged words")
    ap.add_argument("--pass-sweeps", type=int, default=0, help="stream layout: sweeps per pass")
    ap.add_argument("--band-rows", type=int, default=0, help="stream passes: rows per band")
    ap.add_argument("--launch-steps", type=int, default=0,
                    help="steps for the per-launch comparison (default: same as --steps)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--method", default="jacobi", choices=["jacobi", "rb"],
                    help="rb: the same script with red-black Gauss-Seidel iterations instead of "
                         "Jacobi sweeps (one iteration = red then black half-sweep)")
    ap.add_argument("--sweeps-only", action="store_true",
                    help="a step is one SWEEP task of the workload's sweep count (no residuals)")
    ap.add_argument("--launch-only", action="store_true",
                    help="only the per-launch baseline (for counter collection)")
    ap.add_argument("--persistent-only", action="store_true")
    ap.add_argument("--idle-timeout", type=float, default=0.0,
                    help="persistent kernel idle timeout in seconds (0 = engine default)")
    ap.add_argument("--main-only", action="store_true",
                    help="only the timed persistent launch (for counter collection)")
    ap.add_argument("--fold-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="store the traffic of two rocprofv3 counter runs of this workload "
                         "(made with --main-only --calibrate-copy MIB) and exit")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="first run a torch device-to-device copy of MIB MiB (a plain copy "
                         "kernel of known size, to scale HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(json.dumps({"error": "this engine runs on one GPU; --gpus must be 1 "
                          "(the multi-GPU row-band design is described, not built)"}))
        sys.exit(2)

    if args.fold_traffic:
        fold_traffic(args.fold_traffic[0], args.fold_traffic[1], args.workload,
                     args.steps + args.warmup, args.calibrate_copy or 1024)
        return

    if args.calibrate_copy:
        import torch  # before the engine library: one HIP runtime in the process
        n = args.calibrate_copy * (1 << 20) // 4
        x = torch.ones(n, dtype=torch.float32, device="cuda")
        y = torch.empty_like(x)
        y.copy_(x)
        torch.cuda.synchronize()
        del x, y
        torch.cuda.empty_cache()

    w = inputs.make(args.workload)
    if args.method == "rb":
        w.script = [("sweep_rb", s[1]) if s[0] == "sweep" else s for s in w.script]
    if args.sweeps_only:
        w.script = [(sweep_kind(w), w.sweeps)]
    layout = {"auto": pk.PK_LAYOUT_AUTO, "stream": pk.PK_LAYOUT_STREAM,
              "resident": pk.PK_LAYOUT_RESIDENT, "register": pk.PK_LAYOUT_REGISTER}[args.layout]
    barrier = {"auto": pk.PK_BARRIER_AUTO, "flat": pk.PK_BARRIER_FLAT,
               "two_level": pk.PK_BARRIER_TWO_LEVEL, "xcd": pk.PK_BARRIER_XCD}[args.barrier]
    exchange = {"auto": pk.PK_EXCHANGE_AUTO, "barrier": pk.PK_EXCHANGE_BARRIER,
                "neighbor": pk.PK_EXCHANGE_NEIGHBOR, "tagged": pk.PK_EXCHANGE_TAGGED}[args.exchange]
    opts = dict(layout=layout, threads=args.threads, max_blocks=args.max_blocks,
                halo_depth=args.halo, idle_timeout_s=args.idle_timeout, barrier=barrier,
                pass_sweeps=args.pass_sweeps, band_rows=args.band_rows, exchange=exchange)
    step_bytes, sweep_bytes = algorithmic_bytes(w)
    cells_per_step = w.interior_cells * w.sweeps

    if args.launch_only:
        ldt, linfo, _ = measure(w, args.steps, args.warmup, mode=pk.PK_LAUNCH, threads=args.threads,
                                max_blocks=args.max_blocks)
        print(json.dumps({"workload": w.name, "mode": "launch", "steps": args.steps,
                          "us_per_iteration": round(ldt / (w.sweeps * args.steps) * 1e6, 4),
                          "grid_blocks": linfo.grid_blocks, "threads": linfo.threads}), flush=True)
        return

    # persistent engine
    dt, info, info_end = measure(w, args.steps, args.warmup, mode=pk.PK_PERSISTENT, **opts)
    step_us = sorted(measure.step_us)
    value = cells_per_step * args.steps / dt / 1e9
    us_iter = dt / (w.sweeps * args.steps) * 1e6
    kernel_s = info_end.kernel_ms / 1e3
    launch_bytes = step_bytes * (args.steps + args.warmup)
    achieved = launch_bytes / kernel_s / 1e9 if kernel_s > 0 else None

    if args.main_only:
        print(json.dumps({"workload": w.name, "us_per_iteration": round(us_iter, 4),
                          "kernel_ms": info_end.kernel_ms, "steps_in_launch": args.steps + args.warmup}),
              flush=True)
        return
    us_sweep_only = None
    if not args.sweeps_only and sum(1 for t in step_tasks(w) if t[0] == "residual"):
        us_sweep_only = sweep_only(w, args.steps, args.warmup, mode=pk.PK_PERSISTENT, **opts)
    fixed = overheads(w, opts)

    # per-launch baseline, same block count as the persistent grid
    lsteps = args.launch_steps or args.steps
    if args.persistent_only:
        ldt, linfo, lvalue, lsync, lgraph = float("nan"), info, float("nan"), None, None
    else:
        ldt, linfo, _ = measure(w, lsteps, 1, mode=pk.PK_LAUNCH, threads=info.threads,
                                max_blocks=info.grid_blocks)
        lvalue = cells_per_step * lsteps / ldt / 1e9
        lsync = launch_synced(w, min(w.sweeps, 2000), info.threads, info.grid_blocks)
        lgraph = None
        if sweep_kind(w) == "sweep":
            lgraph = launch_graph(w, min(w.sweeps, 10000), info.threads, info.grid_blocks)

    rec = {
        "metric": METRIC,
        "value": round(value, 4),
        "unit": "Gcell-updates/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dt / args.steps * 1e3, 4),
        # each timed step's time on the device clock (its tasks' device times summed)
        "ms_per_step_device": {"min": round(step_us[0] / 1e3, 4),
                               "median": round(step_us[len(step_us) // 2] / 1e3, 4)},
        "us_per_iteration": round(us_iter, 4),
        "us_per_iteration_sweep_task": round(us_sweep_only, 4) if us_sweep_only else round(us_iter, 4),
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
            "residuals_per_step": sum(1 for s in step_tasks(w) if s[0] == "residual"),
            "mode": "persistent",
            "layout": {1: "stream", 2: "resident", 3: "register"}[info.layout],
            "grid_blocks": info.grid_blocks,
            "threads": info.threads,
            "halo_depth": info.halo_depth,
            "band_rows": info.band_rows,
            "barrier": {1: "flat", 2: "two_level", 3: "xcd"}[info.barrier],
            "exchange": {0: None, 1: "barrier", 2: "neighbor", 3: "tagged"}[info.exchange],
            "pass_sweeps": info.pass_sweeps,
        },
        "per_launch": None if args.persistent_only else {
            "value": round(lvalue, 4),
            "us_per_iteration": round(ldt / (w.sweeps * lsteps) * 1e6, 4),
            "us_per_iteration_synced": round(lsync, 4),
            "us_per_iteration_graph": round(lgraph, 4) if lgraph else None,
            "steps": lsteps,
            "grid_blocks": linfo.grid_blocks,
            "kernel_launches_per_step": (2 if args.method == "rb" else 1) * w.sweeps
                                        + 2 * sum(1 for s in step_tasks(w) if s[0] == "residual"),
            "speedup_persistent": round(value / lvalue, 3),
            "speedup_persistent_vs_graph": round(lgraph / us_iter, 3) if lgraph else None,
        },
        "overheads": dict(fixed, tasks_carried=int(info_end.tasks_carried),
                          tasks_done=int(info_end.tasks_done)),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2) if achieved else None,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 5) if achieved else None,
            # the stored counters were taken with the default plan and method
            "traffic": stored_traffic(args.workload, args.steps + args.warmup) if default_plan(args) else None,
            "kernel": "pk_persistent",
            "kernel_ms": round(info_end.kernel_ms, 3),
            "algorithmic_bytes_per_launch": launch_bytes,
            "algorithmic_bytes_per_sweep": sweep_bytes,
        },
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()

"""Shared helpers for the GPU parity tests: run a workload's task script on the
engine and on the CPU oracle, and compare them against the gates.

Gates (field): max |engine - oracle| over every node <= 1e-5 x (max - min of the
oracle field) in fp32, <= 1e-12 x range in fp64. Residual: fp32
|dR| <= 1e-5 R_0 + 1e-9 R_k, fp64 |dR| <= 1e-9 R_k (summation order differs).
"""

from __future__ import annotations

import sys
import time

import numpy as np

import oracle
from iterative_stencil_pde_amd import pk

FIELD_TOL = {np.float32: 1e-5, np.float64: 1e-12}


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def field_gate(got: np.ndarray, ref: np.ndarray):
    """Returns (ok, max_abs_err, tolerance, cells_not_bitwise_equal)."""
    assert got.shape == ref.shape and got.dtype == ref.dtype
    rng = float(ref.max()) - float(ref.min())
    tol = FIELD_TOL[ref.dtype.type] * (rng if rng > 0 else 1.0)
    err = float(np.max(np.abs(got.astype(np.float64) - ref.astype(np.float64))))
    ui = np.uint32 if ref.dtype == np.float32 else np.uint64
    nonbit = int(np.count_nonzero(got.view(ui) != ref.view(ui)))
    return err <= tol, err, tol, nonbit


def residual_gate(got, ref, dtype):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if dtype == np.float32:
        tol = 1e-5 * ref[0] + 1e-9 * np.abs(ref)
    else:
        tol = 1e-9 * np.abs(ref)
    err = np.abs(got - ref)
    return bool(np.all(err <= tol)), float(np.max(err / np.maximum(tol, 1e-300)))


def oracle_until(u, f, h, max_sweeps, every, tol):
    """The early-stop task on the oracle: R of the current field; while R > tol and
    fewer than max_sweeps sweeps are done, min(every, left) sweeps, then R again."""
    r = oracle.residual(u, f=f, h=h)
    done = 0
    while not (r <= tol) and done < max_sweeps:
        k = min(every, max_sweeps - done)
        u, _ = oracle.jacobi(u, k, f=f, h=h)
        done += k
        r = oracle.residual(u, f=f, h=h)
    return u, r, done


def run_engine_pipelined(w, timeout_s: float = 300.0, **opts):
    """Submit the whole script before waiting on anything (the ring allows 64 tasks
    in flight), so the device finds each next task already published: the path on
    which a task is carried in by the previous task's barrier. Steps: "sweep",
    "sweep_rb", "residual", ("until", max, every, tol). No intermediate readbacks."""
    out = {"residuals": [], "results": [], "readbacks": []}
    say(f"[engine, pipelined] {w.name} {w.nx}x{w.ny} opts={opts}")
    with pk.Engine(w.u0, w.f, h=w.h, **opts) as e:
        out["info"] = e.info()
        pending = []
        for step in w.script:
            while True:
                if step[0] == "until":
                    try:
                        t = pk.pk_submit_until(e.h, step[1], step[2], step[3])
                        rc = pk.PK_OK
                    except pk.PkError as ex:
                        rc = ex.status
                else:
                    kind = {"sweep": pk.PK_SWEEP, "sweep_rb": pk.PK_SWEEP_RB,
                            "residual": pk.PK_RESIDUAL}[step[0]]
                    rc, t = pk.pk_submit_status(e.h, kind, step[1] if len(step) > 1 else 0)
                if rc == pk.PK_EBUSY:
                    s0, t0 = pending.pop(0)
                    out["results"].append((s0, e.wait(t0, timeout_s)))
                    continue
                assert rc == pk.PK_OK, rc
                pending.append((step, t))
                break
        for s0, t0 in pending:
            out["results"].append((s0, e.wait(t0, timeout_s)))
        out["residuals"] = [r.residual for s0, r in out["results"] if s0[0] in ("residual", "until")]
        out["final"] = e.readback()
        out["info_end"] = e.info()
    return out


def run_oracle_pipelined(w):
    u = w.u0
    residuals, dones = [], []
    for step in w.script:
        if step[0] == "sweep":
            u, _ = oracle.jacobi(u, step[1], f=w.f, h=w.h)
        elif step[0] == "sweep_rb":
            u, _ = oracle.rbgs(u, step[1], f=w.f, h=w.h)
        elif step[0] == "residual":
            residuals.append(oracle.residual(u, f=w.f, h=w.h))
        elif step[0] == "until":
            u, r, done = oracle_until(u, w.f, w.h, step[1], step[2], step[3])
            residuals.append(r)
            dones.append(done)
    return {"residuals": residuals, "final": u, "readbacks": [], "until_done": dones}


def run_engine_script(w, timeout_s: float = 120.0, **opts):
    """Run ``w.script`` on a fresh engine. Returns dict with residuals, readbacks
    (fields at each readback step), info and per-task results."""
    out = {"residuals": [], "readbacks": [], "results": []}
    say(f"[engine] {w.name} {w.nx}x{w.ny} opts={opts}")
    t0 = time.time()
    with pk.Engine(w.u0, w.f, h=w.h, **opts) as e:
        out["info"] = e.info()
        for step in w.script:
            if step[0] == "sweep":
                r = e.run(pk.PK_SWEEP, step[1], timeout_s)
                out["results"].append(r)
            elif step[0] == "sweep_rb":
                r = e.run(pk.PK_SWEEP_RB, step[1], timeout_s)
                out["results"].append(r)
            elif step[0] == "residual":
                r = e.run(pk.PK_RESIDUAL, 0, timeout_s)
                out["residuals"].append(r.residual)
                out["results"].append(r)
            elif step[0] == "readback":
                out["readbacks"].append(e.readback())
        out["final"] = e.readback()
        out["info_end"] = e.info()
    out["seconds"] = time.time() - t0
    return out


def run_oracle_steps(w):
    """The oracle's answer for a script that may mix Jacobi sweeps ("sweep") and
    red-black iterations ("sweep_rb"), one step at a time."""
    say(f"[oracle, step by step] {w.name}")
    u = w.u0
    residuals, fields = [], []
    for step in w.script:
        if step[0] == "sweep":
            u, _ = oracle.jacobi(u, step[1], f=w.f, h=w.h)
        elif step[0] == "sweep_rb":
            u, _ = oracle.rbgs(u, step[1], f=w.f, h=w.h)
        elif step[0] == "residual":
            residuals.append(oracle.residual(u, f=w.f, h=w.h))
        elif step[0] == "readback":
            fields.append(u.copy())
    return {"residuals": residuals, "readbacks": fields, "final": u}


def run_oracle_script(w):
    """The oracle's answer for ``w.script``: residuals and fields at each readback."""
    if any(s[0] == "sweep_rb" for s in w.script):
        return run_oracle_steps(w)
    say(f"[oracle] {w.name}")
    res_ck = w.residual_checkpoints
    rb_ck = w.readback_checkpoints
    marks = sorted(set(rb_ck) | {w.sweeps})
    fields, residuals = [], []
    u, k, first = w.u0, 0, True
    for mark in marks:
        # residual checkpoints in (k, mark], plus those at 0 in the first segment
        ck = [c - k for c in res_ck if (k < c <= mark) or (first and c == 0)]
        first = False
        u, r = oracle.jacobi(u, mark - k, f=w.f, h=w.h, checkpoints=ck)
        residuals.extend(r.tolist())
        fields.extend(u.copy() for c in rb_ck if c == mark)
        k = mark
    assert len(residuals) == len(res_ck)
    return {"residuals": residuals, "readbacks": fields, "final": u}

"""Decode the engine's device trace (PK_DBG_TRACE) and summarize where a task's
time goes: the work between synchronizations, the wait inside them, and how far
apart the blocks arrive (every block waits for the slowest: "Grid-Wide Barriers
and Persistent Work Queues", "What the barrier buys").

The raw layout is the one ``pk_trace_read`` documents in ``include/pk.h``: per
block, a little-endian uint64 event count, then ``capacity`` records of
{uint64 time, uint32 kind, uint32 aux}; event e sits in record e % capacity.

Usage on a GPU: ``python -m iterative_stencil_pde_amd.trace --workload laplace4096
--sweeps 400`` prints a JSON summary (times in microseconds of the device wall
clock).
"""

from __future__ import annotations

import argparse
import json

import numpy as np

TASK_BEGIN, TASK_END, SYNC_ARRIVE, SYNC_LEAVE, TAG_WAIT, TAG_DONE, PERIOD = 1, 2, 3, 4, 5, 6, 7
KIND_NAMES = {TASK_BEGIN: "task_begin", TASK_END: "task_end", SYNC_ARRIVE: "sync_arrive",
              SYNC_LEAVE: "sync_leave", TAG_WAIT: "tag_wait", TAG_DONE: "tag_done", PERIOD: "period"}
RECORD = np.dtype([("t", "<u8"), ("kind", "<u4"), ("aux", "<u4")])


def block_bytes(capacity: int) -> int:
    return 8 + capacity * RECORD.itemsize


def decode(raw: bytes, grid: int, capacity: int) -> list:
    """Per block, its events in the order it recorded them (the latest `capacity`
    when its ring wrapped), as a structured array (t, kind, aux)."""
    per = block_bytes(capacity)
    if len(raw) < grid * per:
        raise ValueError(f"trace of {len(raw)} bytes, {grid} blocks of {per} expected")
    out = []
    for b in range(grid):
        base = b * per
        count = int.from_bytes(raw[base:base + 8], "little")
        ring = np.frombuffer(raw, dtype=RECORD, count=capacity, offset=base + 8)
        if count <= capacity:
            ev = ring[:count]
        else:
            start = count % capacity
            ev = np.concatenate([ring[start:], ring[:start]])
        out.append(np.array(ev, copy=True))
    return out


def intervals(blocks: list, tick_us: float) -> dict:
    """Durations in us, pooled over blocks:
      work      from a task's start or a sync's departure to the next arrival
      sync_wait from arrival at a grid barrier or neighbour sync to departure
                (also split: barrier_wait, neighbor_wait; the event's aux is 0
                for a grid barrier, 1 for a neighbour sync)
      tag_wait  wave 0's polls for tagged halo words
      period    a tile period, from its start to the next period, tag poll or sync
    and, per synchronization (the i-th of every block), the spread of the blocks'
    arrival times (the slowest block's lead over the fastest)."""
    work, wait, tag, period = [], [], [], []
    by_kind = {0: [], 1: []}
    arrivals = []
    for ev in blocks:
        t_from = None      # start of the current work interval
        t_arrive = None
        a_arrive = 0
        t_tag = None
        t_period = None
        mine = []
        for t, kind, aux in ev:
            t = int(t)
            if kind == TASK_BEGIN:
                t_from = t
            elif kind == SYNC_ARRIVE:
                if t_from is not None:
                    work.append(t - t_from)
                if t_period is not None:
                    period.append(t - t_period)
                    t_period = None
                t_arrive = t
                a_arrive = int(aux)
                mine.append(t)
            elif kind == SYNC_LEAVE:
                if t_arrive is not None:
                    wait.append(t - t_arrive)
                    by_kind.setdefault(a_arrive, []).append(t - t_arrive)
                t_arrive = None
                t_from = t
            elif kind == TAG_WAIT:
                if t_period is not None:
                    period.append(t - t_period)
                    t_period = None
                t_tag = t
            elif kind == TAG_DONE:
                if t_tag is not None:
                    tag.append(t - t_tag)
                t_tag = None
            elif kind == PERIOD:
                if t_period is not None:
                    period.append(t - t_period)
                t_period = t
            elif kind == TASK_END:
                t_from = None
                t_period = None
        arrivals.append(mine)
    n = min((len(a) for a in arrivals), default=0)
    spread = []
    if n and len(arrivals) > 1:
        arr = np.array([a[:n] for a in arrivals], dtype=np.float64)
        spread = list(arr.max(axis=0) - arr.min(axis=0))
    scale = lambda v: np.asarray(v, dtype=np.float64) * tick_us  # noqa: E731
    return {"work": scale(work), "sync_wait": scale(wait), "barrier_wait": scale(by_kind[0]),
            "neighbor_wait": scale(by_kind[1]), "tag_wait": scale(tag), "period": scale(period),
            "arrival_spread": scale(spread)}


def stats(v: np.ndarray, bins: int = 8) -> dict:
    """Count, mean, median, 90th percentile, max and a histogram of equal-width bins."""
    if len(v) == 0:
        return {"count": 0}
    hist, edges = np.histogram(v, bins=bins)
    return {"count": int(len(v)), "mean": round(float(v.mean()), 4), "p50": round(float(np.median(v)), 4),
            "p90": round(float(np.percentile(v, 90)), 4), "max": round(float(v.max()), 4),
            "histogram": {"edges_us": [round(float(x), 4) for x in edges], "counts": [int(c) for c in hist]}}


def summarize(raw: bytes, grid: int, capacity: int, wall_clock_khz: int) -> dict:
    blocks = decode(raw, grid, capacity)
    iv = intervals(blocks, 1e3 / wall_clock_khz)
    total_work, total_wait = float(iv["work"].sum()), float(iv["sync_wait"].sum())
    return {"blocks": grid, "events": int(sum(len(b) for b in blocks)),
            "wrapped_blocks": int(sum(1 for b in blocks if len(b) == capacity)),
            "sync_wait_share": round(total_wait / (total_wait + total_work), 4) if total_work + total_wait else None,
            **{k: stats(v) for k, v in iv.items()}}


def main():
    from iterative_stencil_pde_amd import inputs, pk

    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--workload", default="laplace4096", choices=sorted(inputs.WORKLOADS))
    ap.add_argument("--sweeps", type=int, default=400)
    ap.add_argument("--residual-every", type=int, default=0,
                    help="a RESIDUAL task after every this many sweeps (0: none)")
    ap.add_argument("--exchange", default="auto", choices=["auto", "barrier", "neighbor"],
                    help="how passes (or tile exchanges) meet: the planner's choice, grid barrier, "
                         "or neighbour counters")
    args = ap.parse_args()
    w = inputs.make(args.workload)
    exchange = {"auto": pk.PK_EXCHANGE_AUTO, "barrier": pk.PK_EXCHANGE_BARRIER,
                "neighbor": pk.PK_EXCHANGE_NEIGHBOR}[args.exchange]
    with pk.Engine(w.u0, w.f, h=w.h, flags=pk.PK_DBG_TRACE, exchange=exchange) as e:
        info = e.info()
        # a warm-up task, then the traced stretch, queued ahead of the device (up to
        # 48 tasks in flight, within the 64-slot ring), so that no task waits for
        # the host between them
        pending = []

        def queue(kind, n=0):
            if len(pending) >= 48:
                e.wait(pending.pop(0))
            pending.append(e.submit(kind, n))

        queue(pk.PK_SWEEP, 8)
        every = args.residual_every or args.sweeps
        done = 0
        while done < args.sweeps:
            k = min(every, args.sweeps - done)
            queue(pk.PK_SWEEP, k)
            if args.residual_every:
                queue(pk.PK_RESIDUAL)
            done += k
        queue(pk.PK_EXIT)
        for t in pending:
            e.wait(t)
        raw = e.trace()
        info = e.info()
    out = {"workload": w.name, "sweeps": args.sweeps, "residual_every": args.residual_every,
           "layout": {1: "stream", 2: "resident", 3: "register"}[info.layout], "grid_blocks": info.grid_blocks,
           "threads": info.threads, "halo_depth": info.halo_depth, "pass_sweeps": info.pass_sweeps,
           "exchange": info.exchange,
           **summarize(raw, info.grid_blocks, info.trace_capacity, info.wall_clock_khz)}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

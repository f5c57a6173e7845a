"""GPU tests of the engine's protocol and grid barrier (through the C ABI)."""

import time

import numpy as np
import pytest

import oracle
from iterative_stencil_pde_amd import inputs, pk
from parity import field_gate, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("barrier", [pk.PK_BARRIER_FLAT, pk.PK_BARRIER_TWO_LEVEL, pk.PK_BARRIER_XCD],
                         ids=["flat", "two_level", "xcd"])
def test_stamp_check_correct_barrier(barrier):
    """After each barrier every block sees the stamps all blocks wrote before it
    ("Grid-Wide Barriers", "The barrier is a counter and a generation"; the
    "@persistent" page, "grid_barrier")."""
    w = inputs.laplace_top_edge(4096, 0)
    with pk.Engine(w.u0, None, layout=pk.PK_LAYOUT_STREAM, barrier=barrier) as e:
        info = e.info()
        say(f"  grid={info.grid_blocks} threads={info.threads}")
        r = e.run(pk.PK_STAMP, 20000, 120)
        say(f"  stamp rounds=20000 errors={r.errors} device_us={r.device_us:.0f}")
        assert r.errors == 0 and r.status == 0
        # the field is untouched by barrier-only tasks
        e.run(pk.PK_BARRIER, 1000)
        assert np.array_equal(e.readback(), w.u0)


@pytest.mark.parametrize("barrier", [pk.PK_BARRIER_FLAT, pk.PK_BARRIER_TWO_LEVEL, pk.PK_BARRIER_XCD],
                         ids=["flat", "two_level", "xcd"])
@pytest.mark.parametrize("blocks", [2, 7, 8, 64, 256, 1024])
def test_barrier_only_tasks(blocks, barrier):
    w = inputs.laplace_random_interior(256, 0)
    try:
        eng = pk.Engine(w.u0, None, layout=pk.PK_LAYOUT_STREAM, max_blocks=blocks, threads=256,
                        barrier=barrier)
    except pk.PkError as ex:
        assert ex.status == pk.PK_ELAUNCH
        pytest.skip(f"{blocks} blocks of 256 threads are not co-resident on this device")
    with eng as e:
        r = e.run(pk.PK_BARRIER, 5000)
        r2 = e.run(pk.PK_STAMP, 2000)
        say(f"  blocks={e.info().grid_blocks} barrier_kind={e.info().barrier}: "
            f"{r.device_us / 5000:.3f} us per barrier, stamp errors {r2.errors}")
        assert r2.errors == 0


def test_broken_barrier_negative_control():
    """With the barrier's release/acquire removed (relaxed atomics, no fences:
    every wait still ends and every access is the same as in the correct run),
    blocks can read halo rows that other XCDs' blocks have not yet made visible.
    The field gate is expected to catch that ("Grid-Wide Barriers", "Failure
    modes that only appear at this scale": a barrier of relaxed atomics orders
    progress, not memory traffic)."""
    w = inputs.laplace_random_interior(1024, 0)
    sweeps = 400
    ref, _ = oracle.jacobi(w.u0, sweeps)
    results = {}
    for label, flags, kind in (("correct flat", 0, pk.PK_BARRIER_FLAT),
                               ("correct two-level", 0, pk.PK_BARRIER_TWO_LEVEL),
                               ("correct xcd", 0, pk.PK_BARRIER_XCD),
                               ("broken", pk.PK_DBG_BROKEN_BARRIER, pk.PK_BARRIER_AUTO)):
        with pk.Engine(w.u0, None, layout=pk.PK_LAYOUT_STREAM, flags=flags, barrier=kind) as e:
            e.run(pk.PK_SWEEP, sweeps)
            got = e.readback()
            stamp = e.run(pk.PK_STAMP, 5000).errors
        ok, err, tol, nonbit = field_gate(got, ref)
        say(f"  {label}: max_abs={err:.3e} tol={tol:.3e} non_bitwise={nonbit} stamp_errors={stamp}")
        results[label] = (ok, stamp)
    for label in ("correct flat", "correct two-level", "correct xcd"):
        assert results[label] == (True, 0), label
    # the field gate itself must catch the fence-less barrier; the stamp count is
    # logged above as further evidence
    assert not results["broken"][0], "the fence-less barrier left the field within the parity gate"


def test_protocol_errors_and_ring():
    w = inputs.laplace_top_edge(128, 0)
    per_task = 1000
    with pk.Engine(w.u0, None, layout=pk.PK_LAYOUT_STREAM) as e:
        h = e.h
        # persistent engines refuse the launch-per-sweep baseline
        with pytest.raises(pk.PkError) as ex:
            pk.pk_run_launch_per_iter(h, 1)
        assert ex.value.status == pk.PK_ESTATE
        # unknown task kinds and negative counts
        assert pk.pk_submit_status(h, 99, 0)[0] == pk.PK_EINVAL
        assert pk.pk_submit_status(h, pk.PK_SWEEP, -1)[0] == pk.PK_EINVAL
        assert pk.pk_submit_status(h, pk.PK_SWEEP, pk.PK_TASK_N_MAX + 1)[0] == pk.PK_EINVAL
        # fill the ring: 64 slots, the 65th is refused until the oldest completes
        tickets = []
        status = pk.PK_OK
        for _ in range(64 + 8):
            status, t = pk.pk_submit_status(h, pk.PK_SWEEP, per_task)
            if status != pk.PK_OK:
                break
            tickets.append(t)
        say(f"  accepted {len(tickets)} tasks before status {status}")
        assert status == pk.PK_EBUSY and len(tickets) >= 64
        # readback refuses while tasks are in flight
        out = np.empty_like(w.u0)
        with pytest.raises(pk.PkError) as ex:
            pk.pk_readback(h, out)
        assert ex.value.status == pk.PK_EBUSY
        res = [e.wait(t, 120) for t in tickets]
        assert [r.sweeps_done for r in res] == [per_task * (k + 1) for k in range(len(tickets))]
        # waiting on a ticket never issued
        with pytest.raises(pk.PkError) as ex:
            e.wait(10 ** 6)
        assert ex.value.status == pk.PK_EINVAL
        # readback buffer too small
        with pytest.raises(pk.PkError):
            pk.pk_readback(h, np.empty(10, np.float32))
        t = e.submit(pk.PK_EXIT)
        assert e.wait(t).kind == pk.PK_EXIT
        assert pk.pk_submit_status(h, pk.PK_SWEEP, 1)[0] == pk.PK_ESTATE
        # still readable after EXIT (the kernel has left: an ordinary copy)
        got = e.readback()
        ref, _ = oracle.jacobi(w.u0, per_task * len(tickets))
        assert field_gate(got, ref)[0]
        info = e.info()
        assert info.kernel_ms > 0 and info.kernel_launches == 1


def test_idle_timeout_ends_the_kernel():
    """The kernel leaves by itself when no task comes; the host sees a device
    error, not a hang (forced from the host by simply not submitting)."""
    w = inputs.laplace_harmonic(64, 0)
    with pk.Engine(w.u0, None, idle_timeout_s=0.5) as e:
        e.sweep(10)
        time.sleep(1.5)
        status, _ = pk.pk_submit_status(e.h, pk.PK_SWEEP, 1)
        assert status == pk.PK_ESTATE
        # the field is still there and holds the 10 sweeps
        got = e.readback()
        ref, _ = oracle.jacobi(w.u0, 10)
        assert np.array_equal(got, ref)


def test_grid_that_cannot_be_resident_is_refused():
    """A cooperative grid larger than the device holds is refused, not run
    ("Grid-Wide Barriers", "The residency requirement")."""
    w = inputs.laplace_harmonic(64, 0)
    with pytest.raises(pk.PkError) as ex:
        pk.Engine(w.u0, None, layout=pk.PK_LAYOUT_STREAM, max_blocks=100000, threads=1024)
    assert ex.value.status == pk.PK_ELAUNCH
    # and the device is still usable
    with pk.Engine(w.u0, None) as e:
        e.sweep(3)


def test_launch_mode_rejects_persistent_only_tasks():
    w = inputs.laplace_harmonic(64, 0)
    with pk.Engine(w.u0, None, mode=pk.PK_LAUNCH) as e:
        assert pk.pk_submit_status(e.h, pk.PK_BARRIER, 1)[0] == pk.PK_EINVAL
        assert pk.pk_submit_status(e.h, pk.PK_STAMP, 1)[0] == pk.PK_EINVAL
        us_q = e.launch_per_iter(200, False)
        us_s = e.launch_per_iter(50, True)
        say(f"  launch queued {us_q / 200:.2f} us/sweep, synced {us_s / 50:.2f} us/sweep")
        got = e.readback()
        ref, _ = oracle.jacobi(w.u0, 250)
        assert np.array_equal(got, ref)


# What the planner picks on MI355X (256 CUs, 160 KiB of LDS per block) for the
# five workloads; a change here is a change of the measured plan and should be
# deliberate.
AUTO_PLANS = {
    "laplace64": dict(layout=pk.PK_LAYOUT_RESIDENT, grid_blocks=1),
    "poisson256": dict(layout=pk.PK_LAYOUT_REGISTER, exchange=pk.PK_EXCHANGE_TAGGED, threads=1024),
    "laplace1024": dict(layout=pk.PK_LAYOUT_REGISTER, exchange=pk.PK_EXCHANGE_TAGGED, threads=1024),
    "laplace4096": dict(layout=pk.PK_LAYOUT_STREAM, pass_sweeps=8, threads=512, grid_blocks=256,
                        exchange=pk.PK_EXCHANGE_NEIGHBOR),
    "poisson8192": dict(layout=pk.PK_LAYOUT_STREAM, pass_sweeps=12, threads=512, grid_blocks=256,
                        exchange=pk.PK_EXCHANGE_NEIGHBOR),
}


@pytest.mark.parametrize("name", sorted(AUTO_PLANS))
def test_auto_plan(name):
    w = inputs.make(name)
    with pk.Engine(w.u0, w.f, h=w.h) as e:
        info = e.info()
        e.sweep(2)
    say(f"  {name}: layout={info.layout} G={info.grid_blocks} threads={info.threads} halo={info.halo_depth} "
        f"exchange={info.exchange} k={info.pass_sweeps}")
    for key, want in AUTO_PLANS[name].items():
        assert getattr(info, key) == want, (key, getattr(info, key), want)


@pytest.mark.parametrize("name,layout", [("laplace1024", pk.PK_LAYOUT_STREAM), ("poisson256", pk.PK_LAYOUT_AUTO)])
def test_device_trace(name, layout):
    """PK_DBG_TRACE: every block records its tasks and each synchronization it takes
    part in; the field is unchanged by tracing; the trace is readable only after
    the kernel has left."""
    from iterative_stencil_pde_amd import trace
    w = inputs.make(name)
    with pk.Engine(w.u0, w.f, h=w.h, layout=layout, flags=pk.PK_DBG_TRACE) as e:
        info = e.info()
        assert info.trace_capacity > 0 and info.wall_clock_khz > 0
        e.sweep(40)
        with pytest.raises(pk.PkError) as ex:
            e.trace()
        assert ex.value.status == pk.PK_EBUSY
        got = e.readback()
        e.wait(e.submit(pk.PK_EXIT))
        raw = e.trace()
    ref, _ = oracle.jacobi(w.u0, 40, f=w.f, h=w.h)
    assert np.array_equal(got, ref)
    blocks = trace.decode(raw, info.grid_blocks, info.trace_capacity)
    assert len(blocks) == info.grid_blocks
    for ev in blocks:
        kinds = [int(k) for k in ev["kind"]]
        t = np.asarray(ev["t"], dtype=np.int64)
        assert np.all(np.diff(t) >= 0)  # one block's clock never runs back
        assert kinds.count(trace.TASK_BEGIN) == kinds.count(trace.TASK_END) + 1  # EXIT has no end
        assert kinds.count(trace.SYNC_ARRIVE) == kinds.count(trace.SYNC_LEAVE)
    counts = {len(ev) for ev in blocks}
    syncs = {[int(k) for k in ev["kind"]].count(trace.SYNC_ARRIVE) for ev in blocks}
    assert len(syncs) == 1  # every block takes part in every synchronization
    if info.layout == pk.PK_LAYOUT_STREAM:
        # per pass one grid barrier (40 sweeps in passes of k), plus the task broadcasts
        passes = -(-40 // info.pass_sweeps)
        assert syncs.pop() >= passes
    s = trace.summarize(raw, info.grid_blocks, info.trace_capacity, info.wall_clock_khz)
    say(f"  {name}: layout={info.layout} events/block={sorted(counts)[:3]} work={s['work'].get('mean')} "
        f"wait={s['sync_wait'].get('mean')} tag={s['tag_wait'].get('mean')} period={s['period'].get('mean')}")
    assert s["work"]["count"] > 0


def test_stream_neighbor_counters_replace_the_pass_barriers():
    """Under PK_EXCHANGE_NEIGHBOR the streaming passes of one task meet through
    neighbour counters: 40 sweeps in passes of 4 take 8 neighbour syncs (between
    full-depth passes) and grid barriers only around the task's last two passes
    (the last one sums the residual, one level deeper); the field is the oracle's."""
    from iterative_stencil_pde_amd import trace
    w = inputs.make("laplace1024")
    with pk.Engine(w.u0, w.f, h=w.h, layout=pk.PK_LAYOUT_STREAM, pass_sweeps=4,
                   exchange=pk.PK_EXCHANGE_NEIGHBOR, flags=pk.PK_DBG_TRACE) as e:
        info = e.info()
        assert info.exchange == pk.PK_EXCHANGE_NEIGHBOR
        e.sweep(40)
        got = e.readback()
        e.wait(e.submit(pk.PK_EXIT))
        raw = e.trace()
    ref, _ = oracle.jacobi(w.u0, 40, f=w.f, h=w.h)
    assert np.array_equal(got, ref)
    blocks = trace.decode(raw, info.grid_blocks, info.trace_capacity)
    for ev in blocks:
        kinds = [int(k) for k in ev["kind"]]
        aux = [int(a) for a in ev["aux"]]
        nbr = sum(1 for k, a in zip(kinds, aux) if k == trace.SYNC_ARRIVE and a == 1)
        assert nbr == 8, nbr
        assert kinds.count(trace.SYNC_ARRIVE) == kinds.count(trace.SYNC_LEAVE)
    s = trace.summarize(raw, info.grid_blocks, info.trace_capacity, info.wall_clock_khz)
    say(f"  G={info.grid_blocks} k={info.pass_sweeps} work={s['work'].get('mean')} "
        f"wait={s['sync_wait'].get('mean')}")


def test_trace_needs_the_flag():
    w = inputs.laplace_harmonic(64, 0)
    with pk.Engine(w.u0, None) as e:
        e.sweep(2)
        with pytest.raises(pk.PkError) as ex:
            e.trace()
        assert ex.value.status == pk.PK_ESTATE

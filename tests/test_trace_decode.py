"""The device trace's decoder on synthetic rings (no GPU): record order after a
ring wraps, and the work / wait / spread intervals it derives."""

import numpy as np

from iterative_stencil_pde_amd import trace


def ring(events, capacity):
    """One block's bytes as the device writes them: the count of events ever
    recorded, then the ring (event e in record e % capacity)."""
    rec = np.zeros(capacity, dtype=trace.RECORD)
    for e, (t, kind, aux) in enumerate(events):
        rec[e % capacity] = (t, kind, aux)
    return len(events).to_bytes(8, "little") + rec.tobytes()


def test_decode_keeps_order_and_the_latest_events_after_a_wrap():
    cap = 4
    evs = [(10 * i, trace.PERIOD, i) for i in range(6)]  # 6 events in a ring of 4
    raw = ring(evs[:3], cap) + ring(evs, cap)
    b0, b1 = trace.decode(raw, 2, cap)
    assert [int(x) for x in b0["aux"]] == [0, 1, 2]
    assert [int(x) for x in b1["aux"]] == [2, 3, 4, 5]  # the latest four, oldest first
    assert [int(x) for x in b1["t"]] == [20, 30, 40, 50]


def test_intervals_work_wait_and_arrival_spread():
    T = trace
    # two blocks, one task, two barriers; block 1 arrives 5 ticks later each time
    blk0 = [(0, T.TASK_BEGIN, 1), (100, T.SYNC_ARRIVE, 0), (110, T.SYNC_LEAVE, 0),
            (200, T.SYNC_ARRIVE, 0), (215, T.SYNC_LEAVE, 0), (220, T.TASK_END, 1)]
    blk1 = [(0, T.TASK_BEGIN, 1), (105, T.SYNC_ARRIVE, 0), (110, T.SYNC_LEAVE, 0),
            (210, T.SYNC_ARRIVE, 0), (215, T.SYNC_LEAVE, 0), (220, T.TASK_END, 1)]
    raw = ring(blk0, 8) + ring(blk1, 8)
    iv = T.intervals(T.decode(raw, 2, 8), tick_us=0.01)  # a 100 MHz clock
    assert np.allclose(sorted(iv["work"]), [0.9, 1.0, 1.0, 1.05])
    assert np.allclose(sorted(iv["sync_wait"]), [0.05, 0.05, 0.1, 0.15])
    assert np.allclose(iv["arrival_spread"], [0.05, 0.1])
    assert np.allclose(sorted(iv["barrier_wait"]), [0.05, 0.05, 0.1, 0.15]) and len(iv["neighbor_wait"]) == 0
    s = T.summarize(raw, 2, 8, wall_clock_khz=100000)
    assert s["events"] == 12 and s["wrapped_blocks"] == 0
    assert abs(s["sync_wait_share"] - 0.35 / (0.35 + 3.95)) < 1e-4  # rounded to 4 digits


def test_intervals_tile_periods_and_tag_polls():
    T = trace
    blk = [(0, T.TASK_BEGIN, 1), (0, T.PERIOD, 6), (40, T.TAG_WAIT, 0), (55, T.TAG_DONE, 0),
           (55, T.PERIOD, 6), (95, T.TAG_WAIT, 1), (97, T.TAG_DONE, 1), (97, T.PERIOD, 4),
           (130, T.SYNC_ARRIVE, 0), (140, T.SYNC_LEAVE, 0), (141, T.TASK_END, 1)]
    iv = T.intervals(T.decode(ring(blk, 16), 1, 16), tick_us=1.0)
    assert list(iv["period"]) == [40, 40, 33]
    assert list(iv["tag_wait"]) == [15, 2]
    assert list(iv["work"]) == [130] and list(iv["sync_wait"]) == [10]
    assert len(iv["arrival_spread"]) == 0  # one block: no spread
    st = T.stats(iv["period"], bins=2)
    assert st["count"] == 3 and st["max"] == 40 and sum(st["histogram"]["counts"]) == 3


def test_waits_split_by_synchronization_kind():
    """aux 0 marks a grid barrier, aux 1 a neighbour sync (tile exchanges and the
    streaming passes' neighbour counters)."""
    T = trace
    blk = [(0, T.TASK_BEGIN, 1), (100, T.SYNC_ARRIVE, 1), (104, T.SYNC_LEAVE, 1),
           (200, T.SYNC_ARRIVE, 1), (203, T.SYNC_LEAVE, 1), (300, T.SYNC_ARRIVE, 0),
           (320, T.SYNC_LEAVE, 0), (321, T.TASK_END, 1)]
    iv = T.intervals(T.decode(ring(blk, 16), 1, 16), tick_us=1.0)
    assert list(iv["neighbor_wait"]) == [4, 3] and list(iv["barrier_wait"]) == [20]
    assert sorted(iv["sync_wait"]) == [3, 4, 20]
    assert list(iv["work"]) == [100, 96, 97]

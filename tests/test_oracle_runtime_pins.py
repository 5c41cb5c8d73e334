"""Pins of the runtime oracle (oracle/runtime_ref.py) against values that do
not come from the oracle itself: plain reshapes of a contiguous pool,
hand-worked FIFO chunk sequences, hand-worked scheduler traces and closed
forms of context growth."""

from __future__ import annotations

import itertools

import numpy as np

from oracle import runtime_ref as R


# ------------------------------------------------------------ page movement
def _pool(rng, n, hkv=2):
    return (rng.integers(0, 1 << 16, size=(n, hkv, 16, 128), dtype=np.uint64).astype(np.uint16),
            rng.integers(0, 1 << 16, size=(n, hkv, 16, 128), dtype=np.uint64).astype(np.uint16))


def test_pack_of_all_pages_in_order_is_the_interleaved_pools():
    """Packing every page in order equals stacking K and V along a new axis
    (a plain reshape of the two contiguous pools)."""
    rng = np.random.default_rng(0)
    kp, vp = _pool(rng, 7)
    buf = R.kv_pack_pages(kp, vp, list(range(7)))
    assert np.array_equal(buf, np.stack([kp, vp], axis=1))
    flat = buf.reshape(7, 2, -1)
    assert np.array_equal(flat[:, 0], kp.reshape(7, -1)) and np.array_equal(flat[:, 1], vp.reshape(7, -1))


def test_pack_then_unpack_elsewhere_moves_exactly_those_pages():
    rng = np.random.default_rng(1)
    kp, vp = _pool(rng, 12)
    src, dst = [3, 9, 0, 5], [11, 2, 7, 8]
    buf = R.kv_pack_pages(kp, vp, src)
    k2, v2 = R.kv_unpack_pages(kp, vp, dst, buf)
    for a, b in zip(src, dst):
        assert np.array_equal(k2[b], kp[a]) and np.array_equal(v2[b], vp[a])
    untouched = [p for p in range(12) if p not in dst]
    assert np.array_equal(k2[untouched], kp[untouched]) and np.array_equal(v2[untouched], vp[untouched])


# ------------------------------------------------------------------- FIFO
def test_fifo_hand_worked_sequence():
    """chunk_pages 4, 3 slots: a 10-page evict is cut 4+4+2; the second job
    waits for the first to be fully issued and for a free slot; jobs finish
    in queue order."""
    ops = [("evict", 7, 10), ("evict", 3, 3), ("pump", 2), ("pump", 5), ("poll",), ("pump", 5), ("poll",),
           ("restore", 7, 10), ("pump", 1), ("poll",), ("pump", 9), ("poll",)]
    issued, done = R.offload_fifo(ops, chunk_pages=4, slots=3)
    assert issued == [(7, 1, 0, 4), (7, 1, 4, 4), (7, 1, 8, 2), (3, 1, 0, 3),
                      (7, 2, 0, 4), (7, 2, 4, 4), (7, 2, 8, 2)]
    assert done == [(7, 1), (3, 1), (7, 2)]


def test_fifo_every_page_issued_once_in_order():
    """Random pumps: the chunks of a job tile its pages in order, jobs start
    in queue order, and the finished jobs are a prefix of the queue."""
    rng = np.random.default_rng(2)
    jobs = [(r, int(rng.integers(1, 20))) for r in range(6)]
    ops = [("evict", r, n) for r, n in jobs]
    for _ in range(40):
        ops += [("pump", int(rng.integers(0, 4))), ("poll",)]
    issued, done = R.offload_fifo(ops, chunk_pages=3, slots=2)
    pos, started = {}, []
    for req, kind, first, count in issued:
        assert kind == R.EVICT and first == pos.get(req, 0) and 1 <= count <= 3
        pos[req] = first + count
        if req not in started:
            started.append(req)
    assert started == [r for r, _ in jobs][: len(started)]
    assert done == [(r, R.EVICT) for r, _ in jobs][: len(done)]
    assert all(pos[r] == n for (r, _), (_, n) in zip(done, jobs))
    assert sum(n for _, n in jobs) == sum(c for *_, c in issued)   # 40 rounds issue everything


# -------------------------------------------------------------- scheduler
def test_least_loaded_bucket_balances_counts():
    """Admitting requests one at a time into the least-loaded bucket keeps
    every bucket within one request of every other (exhaustive over small
    starting loads), and ties go to the lowest id."""
    assert R.least_loaded_bucket([2, 1, 1, 3]) == 1
    assert R.least_loaded_bucket([0, 0, 0]) == 0
    for start in itertools.product(range(3), repeat=3):
        loads = list(start)
        for _ in range(12):
            loads[R.least_loaded_bucket(loads)] += 1
        # once the smallest bucket has caught up, the spread never exceeds
        # the initial one and ends at most 1 when the start was balanced
        assert max(loads) - min(loads) <= max(1, max(start) - min(start))
    loads = [0] * 9
    for _ in range(128):
        loads[R.least_loaded_bucket(loads)] += 1
    assert sorted(loads) == [14] * 7 + [15, 15] and loads[:2] == [15, 15]


def test_schedule_without_delay_full_acceptance_closed_form():
    """Every draft accepted, no delay: a request verifies every k+1
    iterations (when t mod (k+1) equals its bucket) and its context grows by
    exactly one token per iteration."""
    k = 3
    arrivals = {0: [(r, 100 + 10 * r, 10 ** 6) for r in range(8)]}
    tr = R.schedule_trace(k, 20, arrivals, accept={}, delayed=False)
    buckets = {rid: b for rid, b, _, _ in tr[0]["batch"]}
    assert sorted(buckets.values()) == [0, 0, 1, 1, 2, 2, 3, 3]
    for it in tr:
        assert it["verify_bucket"] == it["t"] % (k + 1)
        assert len(it["batch"]) == 8
        for rid, b, isv, ctx in it["batch"]:
            assert isv == (b == it["t"] % (k + 1))
            assert ctx == 100 + 10 * rid + it["t"] + 1


def test_schedule_delayed_hand_worked():
    """k = 2, one request in bucket 0, delayed verification, accepting one
    of its drafts at each verify.  t0 verify (no drafts yet) -> t1 waits ->
    t2 draft -> t3 verify (1 draft, accepted) -> t4 waits -> t5 draft -> t6
    verify; its context: 11, -, 12, 13, -, 14, 15."""
    tr = R.schedule_trace(2, 7, {0: [(5, 10, 10 ** 6)]}, accept={(5, 3): 1, (5, 6): 1}, delayed=True)
    seen = [(it["t"], it["batch"]) for it in tr]
    assert seen == [(0, [(5, 0, True, 11)]), (1, []), (2, [(5, 0, False, 12)]), (3, [(5, 0, True, 13)]),
                    (4, []), (5, [(5, 0, False, 14)]), (6, [(5, 0, True, 15)])]


def test_schedule_rejection_rolls_back_and_finishes():
    """k = 3, no delay, one request in bucket 0: verify at t0 (ctx 101, no
    drafts yet), drafts at t1..t3 (ctx 102..104), verify at t4 (ctx 105)
    rejects all three drafts, so the context drops to 102; it then holds
    max_new = 2 committed outputs (1 from t0, 1 from t4) and leaves."""
    tr = R.schedule_trace(3, 6, {0: [(1, 100, 2)]}, accept={(1, 4): 0}, delayed=False)
    assert [b for it in tr for b in it["batch"]][:5] == [(1, 0, True, 101), (1, 0, False, 102), (1, 0, False, 103),
                                                        (1, 0, False, 104), (1, 0, True, 105)]
    assert tr[4]["finished"] == [1] and tr[5]["batch"] == []

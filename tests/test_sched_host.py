"""The native scheduler and offload planner (host code of the library, no GPU
needed) against the runtime oracle.

  * sspec_sched_*: the unified batch scheduler with and without delayed
    verification, driven by random arrivals and the oracle's acceptance
    stub, must produce exactly the oracle's batches (request, bucket, verify
    or draft, context) and finishing order at every iteration;
  * sspec_offload_* in planning-only mode: the chunks issued and the jobs
    reported must be exactly the oracle's FIFO model's.
"""

from __future__ import annotations

import numpy as np
import pytest

from oracle import runtime_ref as R


@pytest.fixture(scope="module")
def S():
    from sparse_self_speculative_amd import sspec
    return sspec


def _drive(S, k, iters, arrivals, max_slots, delayed, rate, seed):
    sched = S.Scheduler(k, max_slots, delayed=delayed)
    req = np.zeros(max_slots, np.int32)
    seq = np.zeros(max_slots, np.int32)
    bk = np.zeros(max_slots, np.int32)
    ctx = np.zeros(max_slots, np.int32)
    sl = np.zeros(max_slots, np.int32)
    trace, prev = [], None

    def resolve(items):
        it, vb, rows = items
        acc = np.zeros(max_slots, np.int32)
        for rid, slot, b in rows:
            if b == vb:
                acc[slot] = R.accept_stub(rid, it, k, rate, seed)
        return sched.resolve(it, acc)

    for t in range(iters):
        for rid, plen, mx in arrivals.get(t, []):
            sched.admit(rid, plen, mx)
        it, vb, n, nv = sched.next(req, seq, bk, ctx, sl)
        assert it == t and vb == t % (k + 1)
        batch = [(int(req[i]), int(bk[i]), bool(bk[i] == vb), int(ctx[seq[i]])) for i in range(n)]
        assert nv == sum(b[2] for b in batch)
        # the selection length the device would hold: the verify's context, cut by rollbacks
        for i in range(n):
            if bk[i] == vb:
                assert sl[seq[i]] == ctx[seq[i]]
            else:
                assert 0 <= sl[seq[i]] <= ctx[seq[i]]
        items = (t, vb, [(int(req[i]), int(seq[i]), int(bk[i])) for i in range(n)])
        if delayed:
            finished = resolve(prev) if prev is not None else []
            prev = items
        else:
            finished = resolve(items)
        trace.append(dict(t=t, verify_bucket=vb, batch=batch, finished=finished))
    return trace


@pytest.mark.parametrize("delayed", [True, False])
@pytest.mark.parametrize("k,rate,seed", [(8, 0.74, 1), (4, 0.3, 2), (2, 1.0, 3), (0, 0.5, 4)])
def test_scheduler_matches_oracle(S, delayed, k, rate, seed):
    rng = np.random.default_rng(seed)
    iters, nreq = 60, 40
    arrivals = {}
    for rid in range(nreq):
        t = int(rng.integers(0, iters // 2))
        arrivals.setdefault(t, []).append((rid, int(rng.integers(20, 3000)), int(rng.integers(1, 25))))
    accept = {(rid, t): R.accept_stub(rid, t, k, rate, seed) for rid in range(nreq) for t in range(iters)}
    want = R.schedule_trace(k, iters, arrivals, accept, delayed=delayed)
    got = _drive(S, k, iters, arrivals, 64, delayed, rate, seed)
    for a, b in zip(got, want):
        assert a == b, f"iteration {a['t']}:\n got  {a}\n want {b}"


def test_scheduler_slots_are_reused_and_buckets_balanced(S):
    """Requests that finish free their slot (the lowest free one is reused)
    and their bucket place (the next arrival joins the emptied bucket)."""
    sched = S.Scheduler(2, 4, delayed=False)
    assert [sched.admit(r, 100, 1) for r in range(3)] == [(0, 0), (1, 1), (2, 2)]
    req, seq, bk, ctx, sl = (np.zeros(4, np.int32) for _ in range(5))
    it, vb, n, nv = sched.next(req, seq, bk, ctx, sl)   # t0: request 0 verifies, max_new 1 -> leaves
    assert (vb, n, nv) == (0, 3, 1)
    assert sched.resolve(0, np.zeros(4, np.int32)) == [0]
    assert sched.admit(7, 50, 5) == (0, 0)              # slot 0 and bucket 0 are free again
    assert sched.query(0)[:2] == (7, 50)


def test_scheduler_rejects_out_of_order_calls(S):
    sched = S.Scheduler(3, 8, delayed=True)
    sched.admit(1, 10, 100)
    buf = [np.zeros(8, np.int32) for _ in range(5)]
    sched.next(*buf)
    sched.next(*buf)
    with pytest.raises(RuntimeError, match="resolve iteration 0"):
        sched.next(*buf)                  # iteration 2 needs iteration 0 resolved
    with pytest.raises(RuntimeError, match="oldest unresolved"):
        sched.resolve(1, np.zeros(8, np.int32))
    sched.resolve(0, np.zeros(8, np.int32))
    sched.next(*buf)
    with pytest.raises(RuntimeError, match="already admitted"):
        sched.admit(1, 10, 100)
    sync = S.Scheduler(3, 1, delayed=False)
    sync.admit(5, 10, 100)
    with pytest.raises(RuntimeError, match="no free slot"):
        sync.admit(6, 10, 100)


@pytest.mark.parametrize("chunk_pages,slots,seed", [(4, 3, 0), (1, 1, 1), (16, 8, 2), (5, 2, 3)])
def test_offload_plan_matches_fifo_model(S, chunk_pages, slots, seed):
    rng = np.random.default_rng(seed)
    eng = S.Offload(None, chunk_pages, slots, dry=True, num_pages=10_000, num_kv_heads=8, host_pages=100_000)
    ops, evicted, restored, nxt = [], [], set(), 0
    for _ in range(200):
        x = rng.random()
        if x < 0.25:
            n = int(rng.integers(1, 40))
            ops.append(("evict", nxt, n))
            evicted.append((nxt, n))
            nxt += 1
        elif x < 0.35 and evicted:
            cand = [e for e in evicted if e[0] not in restored]
            if cand:
                rid, n = cand[int(rng.integers(0, len(cand)))]
                ops.append(("restore", rid, n))
                restored.add(rid)
        elif x < 0.75:
            ops.append(("pump", int(rng.integers(0, 2 * slots + 1))))
        else:
            ops.append(("poll",))
    ops.append(("poll",))
    done = []
    for op in ops:
        if op[0] == "evict":
            eng.evict(op[1], list(range(op[2])))
        elif op[0] == "restore":
            eng.restore(op[1], list(range(op[2])))
        elif op[0] == "pump":
            eng.pump(op[1])
        else:
            done += eng.poll()
    issued_ref, done_ref = R.offload_fifo(ops, chunk_pages, slots)
    assert eng.trace() == issued_ref
    assert done == done_ref


def test_offload_host_errors(S):
    eng = S.Offload(None, 4, 2, dry=True, num_pages=100, num_kv_heads=8, host_pages=10)
    with pytest.raises(RuntimeError, match="host arena full"):
        eng.evict(1, list(range(11)))
    eng.evict(1, list(range(6)))
    with pytest.raises(RuntimeError, match="already has a host copy"):
        eng.evict(1, [7])
    with pytest.raises(RuntimeError, match="outside"):
        eng.evict(2, [100])
    with pytest.raises(RuntimeError, match="no host copy"):
        eng.restore(3, [1])
    with pytest.raises(RuntimeError, match="evicted with 6 pages"):
        eng.restore(1, [1, 2])
    eng.restore(1, list(range(10, 16)))
    with pytest.raises(RuntimeError, match="already being restored"):
        eng.restore(1, list(range(10, 16)))
    eng.pump(100)
    assert eng.poll() == [(1, 1)]       # two slots: 4 + 2 pages of the evict
    eng.pump(100)
    assert eng.poll() == [(1, 2)]
    assert eng.pending() == (0, 0, 10)  # the host copy is free again

"""Plain CPU oracle of the runtime around the attention path: KV offload and
the unified batch scheduler with delayed verification.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  The product path never
calls it and shares no code with it.

Source: the talk-notes page "Accelerating Large-Scale Reasoning Model
Inference with Sparse Self-Speculative Decoding" (MLSys 2026), sections
  * Dynamic KV-Cache management (paper §4.4): requests' KV caches move
    between GPU and host memory asynchronously, in chunks, offloaded and
    loaded back in FIFO order for fairness;
  * Unified batch scheduler (paper §4.2, Fig. 8): requests spread over k+1
    buckets, a new request going to the least-loaded bucket (greedy bin
    packing); each iteration runs k draft buckets and one verify bucket;
  * Delayed verification (paper §4.3, Fig. 9): the verify results of an
    iteration are consumed one iteration later; only the verifying requests
    wait for them, so the host never waits for the GPU inside an iteration.

Pins (tests/test_oracle_runtime_pins.py): pack/unpack against plain
reshapes of a contiguous pool and a round trip; the FIFO model against
hand-worked chunk sequences; the least-loaded assignment against an
exhaustive balance argument and hand-worked traces; the scheduler against
closed forms (context growth with full acceptance, a verify every k+1
iterations per bucket) and hand-worked small traces.

Readings of points the pages leave open (listed in the design notes):
  * chunk = at most chunk_pages pages of ONE request; a job's chunks go out
    in page order; a later job starts only when every chunk of the earlier
    ones has been issued; jobs finish in the order queued;
  * the load of a bucket is its number of live requests; ties go to the
    lowest bucket id;
  * delayed verification: a request that verified in iteration t sits out
    iteration t+1 (its acceptance is not yet known to the host) and resumes
    at t+2 with its rollback applied; the verify bucket of iteration t is
    t mod (k+1);
  * acceptance: a verify of a request with d drafts since its last verify
    accepts a in [0, d] of them (the stub draws a); the request's context
    keeps the verified token plus the a accepted drafts.
"""

from __future__ import annotations

from typing import Dict, List, Sequence, Tuple

import numpy as np

EVICT, RESTORE = 1, 2


# ----------------------------------------------------------- page movement ---

def kv_pack_pages(k_pages: np.ndarray, v_pages: np.ndarray, pages: Sequence[int]) -> np.ndarray:
    """Gather whole pages: [n][2][Hkv][16][d], K block then V block of each
    listed physical page [Dynamic KV-Cache management, §4.4]."""
    out = np.zeros((len(pages), 2) + k_pages.shape[1:], dtype=k_pages.dtype)
    for i, p in enumerate(pages):
        out[i, 0] = k_pages[p]
        out[i, 1] = v_pages[p]
    return out


def kv_unpack_pages(k_pages: np.ndarray, v_pages: np.ndarray, pages: Sequence[int],
                    buf: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Scatter a packed buffer back into the listed pages (copies of the
    pools are returned; the rest of the pools is untouched)."""
    kp, vp = k_pages.copy(), v_pages.copy()
    for i, p in enumerate(pages):
        kp[p] = buf[i, 0]
        vp[p] = buf[i, 1]
    return kp, vp


# ---------------------------------------------------------------- FIFO model ---

def offload_fifo(ops: Sequence[tuple], chunk_pages: int, slots: int) -> Tuple[List[tuple], List[tuple]]:
    """FIFO chunking of evict / restore jobs with chunks finishing at once.

    ops: ("evict", req, n_pages) | ("restore", req, n_pages) |
         ("pump", max_chunks) | ("poll",)
    Returns (issued chunks as (req, kind, first, count) in issue order,
             finished jobs as (req, kind) in report order).
    Chunks finish as soon as a poll runs (the engine's planning-only mode);
    at most `slots` chunks are outstanding between polls.
    """
    jobs: List[dict] = []       # queued, not yet reported
    issued: List[tuple] = []
    done: List[tuple] = []
    outstanding = 0             # chunks issued since the last poll
    for op in ops:
        if op[0] in ("evict", "restore"):
            jobs.append(dict(req=op[1], kind=EVICT if op[0] == "evict" else RESTORE, n=op[2], next=0,
                             open=0))
        elif op[0] == "pump":
            budget = op[1]
            for j in jobs:
                while budget > 0 and j["next"] < j["n"] and outstanding < slots:
                    c = min(chunk_pages, j["n"] - j["next"])
                    issued.append((j["req"], j["kind"], j["next"], c))
                    j["next"] += c
                    j["open"] += 1
                    outstanding += 1
                    budget -= 1
                if j["next"] < j["n"]:
                    break      # a later job waits until this one is fully issued
        elif op[0] == "poll":
            for j in jobs:
                j["open"] = 0
            outstanding = 0
            while jobs and jobs[0]["next"] == jobs[0]["n"]:
                j = jobs.pop(0)
                done.append((j["req"], j["kind"]))
        else:
            raise ValueError(op)
    return issued, done


# ------------------------------------------------------- unified scheduler ---

def _splitmix64(x: int) -> int:
    """SplitMix64 (Steele, Lea and Flood, OOPSLA 2014): one 64-bit counter in,
    one mixed 64-bit value out."""
    m = (1 << 64) - 1
    x = (x + 0x9E3779B97F4A7C15) & m
    x = ((x ^ (x >> 30)) * 0xBF58476D1CE4E5B9) & m
    x = ((x ^ (x >> 27)) * 0x94D049BB133111EB) & m
    return x ^ (x >> 31)


def accept_stub(req_id: int, it: int, k: int, rate: float, seed: int) -> int:
    """The synthetic acceptance test standing in for the model: the verify of
    request req_id in iteration it accepts the leading drafts j = 0, 1, ...
    whose uniform u = (SplitMix64(seed ^ req_id << 40 ^ it << 8 ^ j) >> 11) /
    2^53 lies below `rate`, at most k (the scheduler then clamps to the
    drafts the request holds)."""
    m = (1 << 64) - 1
    base = (seed ^ ((req_id & 0xffffffff) << 40) ^ ((it << 8) & m)) & m
    a = 0
    while a < k:
        u = (_splitmix64(base ^ a) >> 11) * 2.0 ** -53
        if not u < rate:
            break
        a += 1
    return a


def least_loaded_bucket(loads: Sequence[int]) -> int:
    """The bucket with the fewest live requests; the lowest id on ties
    [Unified batch scheduler, §4.2: greedy bin packing of new requests]."""
    best = 0
    for b in range(1, len(loads)):
        if loads[b] < loads[best]:
            best = b
    return best


def schedule_trace(k: int, iters: int, arrivals: Dict[int, List[Tuple[int, int, int]]],
                   accept: Dict[Tuple[int, int], int], delayed: bool = True) -> List[dict]:
    """Run the unified batch scheduler for `iters` iterations.

    arrivals[t]: requests (id, prompt_len, max_new) admitted before
      iteration t's batch is formed.
    accept[(id, t)]: drafts accepted by request id's verify in iteration t
      (clamped to the drafts it holds; missing = all of them).
    A request starts in draft phase with no drafts; in an iteration it runs
    as a verify if its bucket == t mod (k+1), else as a draft.  A draft adds
    one token.  A verify adds one token (the verified one) and resolves the
    drafts made since its last verify: the first `a` stay, the rest are cut.
    With delayed verification the cut is applied at the end of iteration
    t+1 and the request sits out iteration t+1; without it, at the end of
    iteration t.  A request leaves after its verify once its committed
    output reaches max_new tokens; its bucket's load drops then.

    Returns per iteration: dict(t, verify_bucket, batch=[(id, bucket,
    is_verify, ctx_len)], finished=[ids]) where ctx_len is the context the
    attention of that iteration sees (tokens written, current ones included).
    """
    kp1 = k + 1
    loads = [0] * kp1
    live: Dict[int, dict] = {}
    order: List[int] = []
    out = []
    pending: List[Tuple[int, int]] = []     # (id, accepted) resolved at the end of the next iteration
    for t in range(iters):
        for rid, plen, max_new in arrivals.get(t, []):
            b = least_loaded_bucket(loads)
            loads[b] += 1
            live[rid] = dict(bucket=b, ctx=plen, committed=plen, drafts=0, max_new=max_new, out=0,
                             waiting=False)
            order.append(rid)
        vb = t % kp1
        batch = []
        verified = []
        for rid in order:
            r = live.get(rid)
            if r is None or r["waiting"]:
                continue
            if r["bucket"] == vb:
                r["ctx"] += 1
                batch.append((rid, r["bucket"], True, r["ctx"]))
                verified.append(rid)
            else:
                r["ctx"] += 1
                r["drafts"] += 1
                batch.append((rid, r["bucket"], False, r["ctx"]))
        # results of the previous iteration's verifies (delayed) or of this one's
        resolve = pending if delayed else []
        pending = []
        for rid in verified:
            r = live[rid]
            a = min(max(accept.get((rid, t), r["drafts"]), 0), r["drafts"])
            if delayed:
                r["waiting"] = True
                pending.append((rid, a, r["drafts"]))
            else:
                resolve.append((rid, a, r["drafts"]))
        finished = []
        for rid, a, d in resolve:
            r = live[rid]
            r["ctx"] -= d - a
            r["out"] += a + 1
            r["committed"] = r["ctx"]
            r["drafts"] = 0
            r["waiting"] = False
            if r["out"] >= r["max_new"]:
                loads[r["bucket"]] -= 1
                del live[rid]
                finished.append(rid)
        order = [x for x in order if x in live]
        out.append(dict(t=t, verify_bucket=vb, batch=batch, finished=finished))
    return out

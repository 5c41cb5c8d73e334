"""A decode loop driven by the native scheduler with delayed verification, on
the device: per iteration the scheduler forms the batch (slots, buckets,
contexts), the iteration's K/V rows are appended by slot, the unified launch
runs by slot, the acceptance stub draws each verify's accepted drafts on the
device, and the host reads them back one iteration late and resolves them.

Checked against the oracle at every iteration: the batch (request, bucket,
verify or draft, context) and the finished requests equal the runtime
oracle's scheduler trace; the device stub's acceptance counts equal the
oracle's stub; the pools equal the oracle's appends bit for bit; O, LSE and
the selections match the attention oracle (selections up to near-ties)."""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle as O
from oracle import runtime_ref as R
from tests.helpers import assert_attn_close, assert_lse_close, check_topk, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def S():
    from sparse_self_speculative_amd import sspec
    return sspec


def _t16(a):
    return torch.from_numpy(a.view(np.int16)).to(DEV)


def _np16(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("delayed", [True, False])
def test_scheduled_decode_loop(S, delayed):
    say(f"[scheduler loop] delayed={delayed}")
    rng = np.random.default_rng(31 + int(delayed))
    k, hq, hkv, s, rate, seed = 3, 16, 8, 0.1, 0.6, 77
    slots, iters, nreq = 12, 14, 11
    arrivals = {}
    for rid in range(nreq):
        t = 0 if rid < 6 else int(rng.integers(1, 8))
        arrivals.setdefault(t, []).append((rid, int(rng.integers(300, 1400)), int(rng.integers(3, 9))))
    accept = {(rid, t): R.accept_stub(rid, t, k, rate, seed) for rid in range(nreq) for t in range(iters)}
    want = R.schedule_trace(k, iters, arrivals, accept, delayed=delayed)
    # the paged cache: a fixed page list per slot, big enough for any request
    cap_tokens = 1400 + iters + 16
    pps = -(-cap_tokens // 16)
    n_pages = slots * pps
    bt = rng.permutation(n_pages).astype(np.int32).reshape(slots, pps)
    g = torch.Generator().manual_seed(3)

    def bf16(*shape):
        return torch.randn(*shape, generator=g).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)

    kp_h, vp_h = bf16(n_pages, hkv, 16, 128), bf16(n_pages, hkv, 16, 128)
    kp_d, vp_d = _t16(kp_h), _t16(vp_h)
    kv = S.PagedKV(kp_d, vp_d, torch.from_numpy(bt).to(DEV))
    scale = 1 / math.sqrt(128)
    max_ctx = cap_tokens
    sel_stride = O.select_count(max_ctx, s)
    sel_d = torch.zeros(slots, hkv, sel_stride, dtype=torch.int32, device=DEV)
    cnt_d = torch.zeros(slots, dtype=torch.int32, device=DEV)
    ws = S.workspace(S.unified_workspace_size(slots, slots, max_ctx, hq, hkv, k))
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    acc_d = torch.zeros(slots, dtype=torch.int32, device=DEV)
    sched = S.Scheduler(k, slots, delayed=delayed)
    req, seq, bk, ctx, sl = (torch.zeros(slots, dtype=torch.int32).pin_memory() for _ in range(5))
    acc_h = [torch.zeros(slots, dtype=torch.int32).pin_memory() for _ in range(2)]
    sels = [np.zeros((hkv, 0), np.int64) for _ in range(slots)]
    prev = None

    def resolve(p):
        it, vb, items, ev, ah = p
        ev.synchronize()                      # the device's acceptance counts of iteration it
        for rid, slot, b in items:
            if b == vb:
                assert int(ah[slot]) == accept[(rid, it)], f"stub it={it} req={rid}"
        return sched.resolve(it, ah.numpy())

    for t in range(iters):
        for rid, plen, mx in arrivals.get(t, []):
            slot, _ = sched.admit(rid, plen, mx)
            cnt_d[slot] = 0                   # a new request holds no selection yet
            sels[slot] = np.zeros((hkv, 0), np.int64)
        it, vb, n, nv = sched.next(req, seq, bk, ctx, sl)
        items = [(int(req[i]), int(seq[i]), int(bk[i])) for i in range(n)]
        batch = [(rid, b, b == vb, int(ctx[slot])) for rid, slot, b in items]
        if n:
            say(f"   t={t} items={n} verify={nv}")
            seq_d, bk_d = seq[:n].to(DEV, non_blocking=True), bk[:n].to(DEV, non_blocking=True)
            ctx_d, sl_d = ctx.to(DEV, non_blocking=True), sl.to(DEV, non_blocking=True)
            isv = np.array([b == vb for _, _, b in items])
            nrows = np.where(isv, k + 1, 1)
            rows = int(nrows.sum())
            k_new, v_new, q = bf16(rows, hkv, 128), bf16(rows, hkv, 128), bf16(rows, hq, 128)
            S.kv_append_slots(kv, _t16(k_new), _t16(v_new), seq_d, ctx_d, bk_d, vb, n, k, err=err)
            out = torch.empty(rows, hq, 128, dtype=torch.bfloat16, device=DEV)
            lse = torch.empty(rows, hq, dtype=torch.float32, device=DEV)
            S.unified_attn_slots(kv, _t16(q).view(torch.bfloat16), seq_d, ctx_d, bk_d, vb, n, slots, max_ctx, hq,
                                 k, s, scale, sel_d, sel_stride, cnt_d, sl_d, out, lse, ws)
            if nv:
                req_d = req[:n].to(DEV, non_blocking=True)
                S.accept_stub(req_d, seq_d, bk_d, vb, n, k, it, rate, seed, slots, acc_d)
            ah = acc_h[t % 2]
            ah.copy_(acc_d, non_blocking=True)
            ev = torch.cuda.Event()
            ev.record()
            # the oracle's view of the same iteration (blocking: test only)
            slots_i = np.array([slot for _, slot, _ in items])
            ctx_i = ctx.numpy()[slots_i].astype(np.int64)
            kp_h, vp_h, skipped = O.kv_append(kp_h, vp_h, bt[slots_i], k_new, v_new, ctx_i, nrows)
            assert not skipped
            torch.cuda.synchronize()
            assert int(err.item()) == 0 and S.read_device_error(ws) == 0
            assert np.array_equal(_np16(kp_d), kp_h) and np.array_equal(_np16(vp_d), vp_h), f"t={t}: pools"
            sel_len_i = sl.numpy()[slots_i].astype(np.int64)
            o_ref, l_ref, sel_ref, _ = O.unified_step(O.bf16_to_f64(q), kp_h, vp_h, bt[slots_i], ctx_i, isv, k, s,
                                                      scale, [sels[x] for x in slots_i], sel_len_i)
            assert_attn_close(O.bf16_to_f64(_np16(out.view(torch.int16))), o_ref, f"loop O t={t}")
            assert_lse_close(lse.cpu().numpy(), l_ref, f"loop LSE t={t}")
            sel_h, cnt_h = sel_d.cpu().numpy(), cnt_d.cpu().numpy()
            off = np.concatenate([[0], np.cumsum(nrows)])
            for j in np.nonzero(isv)[0]:
                x = slots_i[j]
                kc = O.gather_kv(kp_h, bt[x], int(ctx_i[j]), 16)
                vc = O.gather_kv(vp_h, bt[x], int(ctx_i[j]), 16)
                _, lse_r, lg_r = O.verify_attention(O.bf16_to_f64(q[off[j]: off[j + 1]]), kc, vc, scale)
                S_ref = O.pillar_scores(lg_r, lse_r, hkv)
                for h in range(hkv):
                    check_topk(sel_h[x, h], int(cnt_h[x]), S_ref[h], sel_ref[j][h], f"t={t} slot={x} h={h}")
                sels[x] = sel_h[x, :, : cnt_h[x]].astype(np.int64)
            cur = (it, vb, items, ev, ah)
        else:
            ev = torch.cuda.Event()
            ev.record()
            cur = (it, vb, items, ev, acc_h[t % 2])
        if delayed:
            finished = resolve(prev) if prev is not None else []
            prev = cur
        else:
            finished = resolve(cur)
        got = dict(t=t, verify_bucket=vb, batch=batch, finished=finished)
        assert got == want[t], f"iteration {t}:\n got  {got}\n want {want[t]}"

"""KV offload on the device: the page movers bit for bit against the oracle,
an evict -> overwrite -> restore round trip that leaves attention outputs
bitwise unchanged, and the engine's transfers running on a side stream
beside unified launches without disturbing them."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle as O
from oracle import runtime_ref as R
from sspec_workload import cycle_state, make_workload, pack_rows
from tests.helpers import say

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def S():
    from sparse_self_speculative_amd import sspec
    return sspec


def _u16(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _pools(n_pages, hkv, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    kp = torch.randn(n_pages, hkv, 16, 128, generator=g).to(torch.bfloat16)
    vp = torch.randn(n_pages, hkv, 16, 128, generator=g).to(torch.bfloat16)
    return kp.to(DEV), vp.to(DEV)


@pytest.mark.parametrize("hkv,n", [(8, 37), (2, 5), (1, 1)])
def test_pack_unpack_bit_exact(S, hkv, n):
    say(f"[offload] pack/unpack hkv={hkv} n={n}")
    kp, vp = _pools(64, hkv, 3 + hkv)
    kv = S.PagedKV(kp, vp, torch.zeros(1, 1, dtype=torch.int32, device=DEV))
    rng = np.random.default_rng(n)
    src = rng.permutation(64)[:n].astype(np.int32)
    dst = rng.permutation(64)[:n].astype(np.int32)
    page_el = hkv * 16 * 128
    buf = torch.full((n, 2, hkv, 16, 128), float("nan"), dtype=torch.bfloat16, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    S.kv_pack_pages(kv, torch.from_numpy(src).to(DEV), buf, err=err)
    torch.cuda.synchronize()
    kp_h, vp_h = _u16(kp), _u16(vp)
    assert int(err.item()) == 0
    assert np.array_equal(_u16(buf), R.kv_pack_pages(kp_h, vp_h, src))
    S.kv_unpack_pages(kv, torch.from_numpy(dst).to(DEV), buf, err=err)
    torch.cuda.synchronize()
    k2, v2 = R.kv_unpack_pages(kp_h, vp_h, dst, R.kv_pack_pages(kp_h, vp_h, src))
    assert np.array_equal(_u16(kp), k2) and np.array_equal(_u16(vp), v2)
    assert page_el * 2 * 2 == S.offload_page_bytes(hkv)


def test_pack_skips_bad_pages_and_flags(S):
    say("[offload] bad page ids")
    kp, vp = _pools(8, 2, 1)
    kv = S.PagedKV(kp, vp, torch.zeros(1, 1, dtype=torch.int32, device=DEV))
    pages = torch.tensor([3, -1, 8, 5], dtype=torch.int32, device=DEV)
    buf = torch.zeros(4, 2, 2, 16, 128, dtype=torch.bfloat16, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    S.kv_pack_pages(kv, pages, buf, err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == S.DEV_ERR["PAGE_RANGE"]
    ref = R.kv_pack_pages(_u16(kp), _u16(vp), [3, 5])
    got = _u16(buf)
    assert np.array_equal(got[[0, 3]], ref) and not got[[1, 2]].any()


def _engine(S, kv, hkv, chunk, slots, host_pages, side):
    pb = S.offload_page_bytes(hkv)
    staging = torch.empty(slots * chunk * pb, dtype=torch.uint8, device=DEV)
    host = torch.empty(S.offload_host_bytes(hkv, chunk, slots, host_pages), dtype=torch.uint8, pin_memory=True)
    return S.Offload(kv, chunk, slots, staging=staging, host=host, side_stream=side)


def _drain(eng, want):
    done = []
    for _ in range(100000):
        eng.pump(64)
        done += eng.poll()
        if len(done) >= want:
            return done
    raise AssertionError(f"offload did not finish: {done}")


def test_evict_restore_round_trip_keeps_attention_exact(S):
    """Evict two requests' pages to host memory, overwrite those device pages,
    restore the caches into other free pages and point the block table at
    them: the unified launch then gives bitwise the same outputs."""
    say("[offload] evict -> overwrite -> restore round trip")
    lengths = [900, 2100, 700, 1500, 1200]
    hq, hkv, k, s = 16, 8, 4, 0.1
    w = make_workload(dict(hq=hq, hkv=hkv, k=k, s=s, batch=len(lengths)), seed=21, lengths=lengths)
    n0 = w.k_pages.shape[0]
    spare = 300
    kp = torch.cat([w.k_pages, torch.zeros(spare, *w.k_pages.shape[1:], dtype=torch.bfloat16)]).to(DEV)
    vp = torch.cat([w.v_pages, torch.zeros(spare, *w.v_pages.shape[1:], dtype=torch.bfloat16)]).to(DEV)
    bt = w.block_table.clone().to(DEV)
    kv = S.PagedKV(kp, vp, bt)
    B = w.batch
    max_ctx = int(w.caps.max())
    sel_stride = O.select_count(max_ctx, s)
    mv = int(np.bincount(w.bucket_ids).max())

    def run():
        ws = S.workspace(S.unified_workspace_size(B, mv, max_ctx, hq, hkv, k))
        sel = torch.zeros(B, hkv, sel_stride, dtype=torch.int32, device=DEV)
        cnt = torch.zeros(B, dtype=torch.int32, device=DEV)
        sl = torch.zeros(B, dtype=torch.int32, device=DEV)
        outs = []
        for t in range(k + 1):
            vb, isv, ctx, step = cycle_state(w, t)
            q = pack_rows(w, isv, step, DEV)
            out = torch.empty_like(q)
            lse = torch.empty(q.shape[0], hq, dtype=torch.float32, device=DEV)
            S.unified_attn(kv, q, torch.from_numpy(ctx.astype(np.int32)).to(DEV),
                           torch.from_numpy(w.bucket_ids).to(DEV), vb, B, mv, max_ctx, hq, k, s, w.sm_scale,
                           sel, sel_stride, cnt, sl, out, lse, ws)
            outs.append((out.clone(), lse.clone()))
        torch.cuda.synchronize()
        assert S.read_device_error(ws) == 0
        return outs, sel.clone()

    before, sel_before = run()
    side = torch.cuda.Stream()
    eng = _engine(S, kv, hkv, chunk=7, slots=3, host_pages=400, side=side)
    npg = [-(-int(w.caps[r]) // 16) for r in range(B)]
    movers = [1, 3]
    old = {r: bt[r, : npg[r]].cpu().numpy().copy() for r in movers}
    for r in movers:
        eng.evict(r, old[r])
    ev = torch.cuda.Event()
    ev.record()
    eng.pump(64, after_event=ev)
    assert sorted(_drain(eng, 2)) == [(1, S.OFFLOAD_EVICT), (3, S.OFFLOAD_EVICT)]
    side.synchronize()
    g = torch.Generator(device=DEV).manual_seed(5)
    for r in movers:                      # the freed pages get reused by someone else
        idx = torch.from_numpy(old[r].astype(np.int64)).to(DEV)
        kp[idx] = torch.randn(len(idx), *kp.shape[1:], generator=g, device=DEV).to(torch.bfloat16)
        vp[idx] = torch.randn(len(idx), *vp.shape[1:], generator=g, device=DEV).to(torch.bfloat16)
    free = list(range(n0, n0 + spare))
    new = {}
    for r in movers:
        new[r], free = np.array(free[: npg[r]], np.int32), free[npg[r]:]
        eng.restore(r, new[r])
    ev.record()
    eng.pump(64, after_event=ev)
    assert sorted(_drain(eng, 2)) == [(1, S.OFFLOAD_RESTORE), (3, S.OFFLOAD_RESTORE)]
    side.synchronize()
    for r in movers:
        bt[r, : npg[r]] = torch.from_numpy(new[r]).to(DEV)
    after, sel_after = run()
    for (o0, l0), (o1, l1) in zip(before, after):
        assert torch.equal(o0, o1) and torch.equal(l0, l1)
    assert torch.equal(sel_before, sel_after)
    assert eng.pending() == (0, 0, 400)
    trace = eng.trace()
    assert trace == R.offload_fifo([("evict", 1, npg[1]), ("evict", 3, npg[3]), ("pump", 10 ** 6), ("poll",),
                                    ("restore", 1, npg[1]), ("restore", 3, npg[3]), ("pump", 10 ** 6), ("poll",)],
                                   7, 10 ** 6)[0]
    eng.close()


def test_offload_beside_unified_launches(S):
    """Evictions and restores of a separate cold pool run on a side stream
    while unified launches run on the main stream: the launches' outputs are
    bitwise those of launches with no transfers, and the moved pages arrive
    exact."""
    say("[offload] transfers beside unified launches")
    lengths = [3000, 2500, 4000, 1800, 2200, 3300, 2700, 1500]
    hq, hkv, k, s = 32, 8, 8, 0.05
    w = make_workload(dict(hq=hq, hkv=hkv, k=k, s=s, batch=len(lengths)), seed=22, lengths=lengths)
    kv = S.PagedKV(w.k_pages.to(DEV), w.v_pages.to(DEV), w.block_table.to(DEV))
    B, max_ctx = w.batch, int(w.caps.max())
    sel_stride = O.select_count(max_ctx, s)
    mv = int(np.bincount(w.bucket_ids).max())
    cold_k, cold_v = _pools(600, hkv, 9)
    cold_ref = (_u16(cold_k), _u16(cold_v))
    cold = S.PagedKV(cold_k, cold_v, torch.zeros(1, 1, dtype=torch.int32, device=DEV))

    def launches(eng=None):
        ws = S.workspace(S.unified_workspace_size(B, mv, max_ctx, hq, hkv, k))
        sel = torch.zeros(B, hkv, sel_stride, dtype=torch.int32, device=DEV)
        cnt = torch.zeros(B, dtype=torch.int32, device=DEV)
        sl = torch.zeros(B, dtype=torch.int32, device=DEV)
        outs, done = [], []
        for t in range(3 * (k + 1)):
            vb, isv, ctx, step = cycle_state(w, t)
            q = pack_rows(w, isv, step, DEV)
            out = torch.empty_like(q)
            lse = torch.empty(q.shape[0], hq, dtype=torch.float32, device=DEV)
            S.unified_attn(kv, q, torch.from_numpy(ctx.astype(np.int32)).to(DEV),
                           torch.from_numpy(w.bucket_ids).to(DEV), vb, B, mv, max_ctx, hq, k, s, w.sm_scale,
                           sel, sel_stride, cnt, sl, out, lse, ws)
            if eng is not None:
                if t == 0:
                    for j in range(6):
                        eng.evict(j, list(range(100 * j, 100 * j + 100)))
                if t == k + 1:
                    for j in range(6):   # back into the other half of each block, reversed
                        eng.restore(j, list(range(100 * j + 99, 100 * j - 1, -1)))
                eng.pump(4)   # the cold pool is not touched by the main stream: no wait
                done += eng.poll()
            outs.append((out, lse))
        torch.cuda.synchronize()
        assert S.read_device_error(ws) == 0
        return outs, done

    ref, _ = launches()
    side = torch.cuda.Stream()
    eng = _engine(S, cold, hkv, chunk=16, slots=4, host_pages=700, side=side)
    got, done = launches(eng)
    done += _drain(eng, 12 - len(done)) if len(done) < 12 else []
    side.synchronize()
    assert done == [(j, S.OFFLOAD_EVICT) for j in range(6)] + [(j, S.OFFLOAD_RESTORE) for j in range(6)]
    for (o0, l0), (o1, l1) in zip(ref, got):
        assert torch.equal(o0, o1) and torch.equal(l0, l1)
    kh, vh = _u16(cold_k), _u16(cold_v)
    for j in range(6):
        for i in range(100):
            assert np.array_equal(kh[100 * j + 99 - i], cold_ref[0][100 * j + i])
            assert np.array_equal(vh[100 * j + 99 - i], cold_ref[1][100 * j + i])
    eng.close()

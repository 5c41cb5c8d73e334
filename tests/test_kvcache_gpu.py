"""Paged KV append and rollback (sspec_kv_append, sspec_kv_rollback) against
the oracle, bit for bit, and a decode loop that chains them with the
unified attention.

  * append: random 16-bit patterns (NaN and inf patterns included) for the
    new rows, unified batches with verifying and drafting requests, rows
    whose position or page is out of range skipped with their error bits;
  * rollback: accepted counts across [0, k] and beyond (clamped);
  * decode loop: every iteration appends the current tokens' K/V, runs the
    unified launch (compared with the oracle on the oracle's own copy of the
    pools), and after each verify rolls the verifying requests back to a
    random number of accepted drafts, for two full bucket cycles.
Every case prints its name before touching the GPU.
"""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle as O
from tests.helpers import assert_attn_close, assert_lse_close, check_topk, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def S():
    from sparse_self_speculative_amd import sspec
    return sspec


def _bits(rng, *shape):
    return rng.integers(0, 1 << 16, size=shape, dtype=np.uint64).astype(np.uint16)


def _t16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV)


def _np16(t):
    return t.cpu().numpy().view(np.uint16)


def _paged(rng, B, caps, hkv, extra_pages=0):
    npg = -(-np.asarray(caps) // 16)
    total = int(npg.sum()) + extra_pages
    perm = rng.permutation(total).astype(np.int32)
    bt = np.zeros((B, int(npg.max())), np.int32)
    off = 0
    for r in range(B):
        bt[r, : npg[r]] = perm[off: off + npg[r]]
        off += int(npg[r])
    return _bits(rng, total, hkv, 16, 128), _bits(rng, total, hkv, 16, 128), bt


@pytest.mark.parametrize("B,hkv,k,vb", [(12, 8, 8, 2), (20, 2, 16, 0), (7, 8, 0, 1), (9, 4, 4, 7)])
def test_kv_append_bit_exact(S, B, hkv, k, vb):
    say(f"[kv append] B={B} hkv={hkv} k={k} verify_bucket={vb}")
    rng = np.random.default_rng(B * 100 + k)
    buckets = rng.integers(0, k + 1, size=B).astype(np.int32)
    isv = buckets == vb
    nrows = O.unified_rows(isv, k)
    ctx = rng.integers(k + 1, 900, size=B).astype(np.int32)
    kp, vp, bt = _paged(rng, B, ctx + 5, hkv)
    rows = int(nrows.sum())
    k_new, v_new = _bits(rng, rows, hkv, 128), _bits(rng, rows, hkv, 128)
    kp_d, vp_d = _t16(kp), _t16(vp)
    kv = S.PagedKV(kp_d, vp_d, torch.from_numpy(bt).to(DEV))
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    S.kv_append(kv, _t16(k_new), _t16(v_new), torch.from_numpy(ctx).to(DEV), torch.from_numpy(buckets).to(DEV),
                vb, B, k, err=err)
    torch.cuda.synchronize()
    ref_k, ref_v, skipped = O.kv_append(kp, vp, bt, k_new, v_new, ctx, nrows)
    assert not skipped and int(err.item()) == 0
    assert np.array_equal(_np16(kp_d), ref_k) and np.array_equal(_np16(vp_d), ref_v)


def test_kv_append_bad_rows_flag_and_skip(S):
    """A request whose context lies beyond its block-table row (CTX_RANGE) and
    one whose page is outside the pool (PAGE_RANGE): their rows are skipped,
    every other row lands, and the error bits are set."""
    say("[kv append] bad rows")
    rng = np.random.default_rng(3)
    B, hkv, k, vb = 6, 8, 8, 1
    buckets = np.array([1, 0, 1, 2, 0, 1], np.int32)
    isv = buckets == vb
    nrows = O.unified_rows(isv, k)
    ctx = np.array([200, 300, 150, 64, 500, 77], np.int32)
    kp, vp, bt = _paged(rng, B, ctx + 3, hkv)
    ctx_bad = ctx.copy()
    ctx_bad[3] = bt.shape[1] * 16 + 40            # past the block table's row
    bt_bad = bt.copy()
    bt_bad[5, (77 - 1) // 16] = kp.shape[0] + 3   # the page of request 5's verify rows (68..76) outside the pool
    rows = int(nrows.sum())
    k_new, v_new = _bits(rng, rows, hkv, 128), _bits(rng, rows, hkv, 128)
    kp_d, vp_d = _t16(kp), _t16(vp)
    kv = S.PagedKV(kp_d, vp_d, torch.from_numpy(bt_bad).to(DEV))
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    S.kv_append(kv, _t16(k_new), _t16(v_new), torch.from_numpy(ctx_bad).to(DEV), torch.from_numpy(buckets).to(DEV),
                vb, B, k, err=err)
    torch.cuda.synchronize()
    ref_k, ref_v, skipped = O.kv_append(kp, vp, bt_bad, k_new, v_new, ctx_bad, nrows)
    assert skipped
    assert int(err.item()) == S.DEV_ERR["CTX_RANGE"] | S.DEV_ERR["PAGE_RANGE"]
    assert np.array_equal(_np16(kp_d), ref_k) and np.array_equal(_np16(vp_d), ref_v)


def test_kv_rollback_bit_exact(S):
    say("[kv rollback]")
    rng = np.random.default_rng(4)
    B, k, vb = 300, 8, 5
    buckets = rng.integers(0, k + 1, size=B).astype(np.int32)
    isv = buckets == vb
    ctx = rng.integers(k + 1, 40000, size=B).astype(np.int32)
    sel_len = np.where(rng.random(B) < 0.5, ctx, ctx - rng.integers(0, 12, size=B)).astype(np.int32)
    acc = rng.integers(-3, k + 4, size=B).astype(np.int32)
    ctx_d, sl_d = torch.from_numpy(ctx.copy()).to(DEV), torch.from_numpy(sel_len.copy()).to(DEV)
    S.kv_rollback(torch.from_numpy(buckets).to(DEV), vb, torch.from_numpy(acc).to(DEV), B, k, ctx_d, sl_d)
    torch.cuda.synchronize()
    ref_ctx, ref_sl = O.kv_rollback(ctx, sel_len, isv, acc, k)
    assert np.array_equal(ctx_d.cpu().numpy(), ref_ctx) and np.array_equal(sl_d.cpu().numpy(), ref_sl)


def test_decode_loop_append_attend_rollback(S):
    """Two full bucket cycles of a self-speculative decode loop on the device:
    append the iteration's K/V (a verifying request rewrites its last
    committed token and its k drafts, a drafting request writes its one
    token), unified attention, then the rollback of the verifying requests
    to a random number of accepted drafts.  The oracle runs the same loop
    on its own copy of the pools; after every iteration the pools must be
    bitwise equal, O and LSE within tolerance, the selections equal up to
    near-ties, and ctx_lens / sel_len / sel_count exactly equal.  The loop
    starts with no selection (sel_count 0, sel_len 0): a draft before its
    request's first verify attends to its whole context."""
    say("[decode loop] append -> unified attention -> rollback")
    rng = np.random.default_rng(7)
    B, hq, hkv, k, s = 10, 16, 8, 4, 0.1
    kp1 = k + 1
    scale = 1 / math.sqrt(128)
    base = rng.integers(200, 1600, size=B).astype(np.int64)   # committed tokens; the bonus token is not written yet
    iters = 2 * kp1
    caps = base + iters * kp1 + 1
    kp_h, vp_h, bt = _paged(rng, B, caps, hkv)
    # random bf16 values (finite) for the initial cache contents and new rows
    def bf16(*shape):
        return torch.randn(*shape, generator=gen).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    gen = torch.Generator().manual_seed(11)
    kp_h[:] = bf16(*kp_h.shape)
    vp_h[:] = bf16(*vp_h.shape)
    buckets = (np.arange(B) % kp1).astype(np.int32)
    max_ctx = int(caps.max())
    sel_stride = math.ceil(s * max_ctx)
    kp_d, vp_d = _t16(kp_h), _t16(vp_h)
    kv = S.PagedKV(kp_d, vp_d, torch.from_numpy(bt).to(DEV))
    bk_d = torch.from_numpy(buckets).to(DEV)
    sel_d = torch.zeros(B, hkv, sel_stride, dtype=torch.int32, device=DEV)
    cnt_d = torch.zeros(B, dtype=torch.int32, device=DEV)
    sl_d = torch.zeros(B, dtype=torch.int32, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    ws = S.workspace(S.unified_workspace_size(B, B, max_ctx, hq, hkv, k))
    sels = [np.zeros((hkv, 0), np.int64) for _ in range(B)]
    sel_len = np.zeros(B, np.int64)
    for t in range(iters):
        vb = t % kp1
        isv = buckets == vb
        step = (t - buckets) % kp1                           # 0: verify, j: draft step j
        ctx = np.where(isv, base + kp1, base + step).astype(np.int64)
        nrows = O.unified_rows(isv, k)
        rows = int(nrows.sum())
        k_new, v_new = bf16(rows, hkv, 128), bf16(rows, hkv, 128)
        q = bf16(rows, hq, 128)
        ctx_d = torch.from_numpy(ctx.astype(np.int32)).to(DEV)
        S.kv_append(kv, _t16(k_new), _t16(v_new), ctx_d, bk_d, vb, B, k, err=err)
        kp_h, vp_h, skipped = O.kv_append(kp_h, vp_h, bt, k_new, v_new, ctx, nrows)
        assert not skipped
        out = torch.empty(rows, hq, 128, dtype=torch.bfloat16, device=DEV)
        lse = torch.empty(rows, hq, dtype=torch.float32, device=DEV)
        S.unified_attn(kv, _t16(q).view(torch.bfloat16).view(rows, hq, 128), ctx_d, bk_d, vb, B, B, max_ctx, hq, k,
                       s, scale, sel_d, sel_stride, cnt_d, sl_d, out, lse, ws)
        torch.cuda.synchronize()
        flags = (int(err.item()), S.read_device_error(ws))
        assert flags == (0, 0), f"t={t}: append / unified device error bits {flags}"
        assert np.array_equal(_np16(kp_d), kp_h) and np.array_equal(_np16(vp_d), vp_h), f"t={t}: pools differ"
        o_ref, l_ref, sel_ref, sl_ref = O.unified_step(O.bf16_to_f64(q), kp_h, vp_h, bt, ctx, isv, k, s, scale,
                                                       sels, sel_len)
        assert_attn_close(O.bf16_to_f64(_np16(out.view(torch.int16))), o_ref, f"loop O t={t}")
        assert_lse_close(lse.cpu().numpy(), l_ref, f"loop LSE t={t}")
        sel_h, cnt_h, sl_h = sel_d.cpu().numpy(), cnt_d.cpu().numpy(), sl_d.cpu().numpy()
        assert np.array_equal(sl_h, sl_ref), f"t={t}: sel_len"
        off = np.concatenate([[0], np.cumsum(nrows)])
        for r in np.nonzero(isv)[0]:
            kc = O.gather_kv(kp_h, bt[r], int(ctx[r]), 16)
            vc = O.gather_kv(vp_h, bt[r], int(ctx[r]), 16)
            _, lse_r, lg_r = O.verify_attention(O.bf16_to_f64(q[off[r]: off[r + 1]]), kc, vc, scale)
            S_ref = O.pillar_scores(lg_r, lse_r, hkv)
            for h in range(hkv):
                check_topk(sel_h[r, h], int(cnt_h[r]), S_ref[h], sel_ref[r][h], f"loop t={t} r={r} h={h}")
            # carry the device's selection (equal up to near-ties) into the oracle's state
            sels[r] = sel_h[r, :, : cnt_h[r]].astype(np.int64)
        sel_len = sl_ref
        if isv.any():
            acc = rng.integers(0, kp1, size=B).astype(np.int32)
            S.kv_rollback(bk_d, vb, torch.from_numpy(acc).to(DEV), B, k, ctx_d, sl_d)
            torch.cuda.synchronize()
            new_ctx, new_sl = O.kv_rollback(ctx, sel_len, isv, acc, k)
            assert np.array_equal(ctx_d.cpu().numpy(), new_ctx) and np.array_equal(sl_d.cpu().numpy(), new_sl)
            base = np.where(isv, new_ctx, base)
            sel_len = new_sl

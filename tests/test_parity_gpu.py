"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Sizes span several tiles, splits and a ragged tail while the oracle still
finishes in seconds.  Every case prints its name before touching the GPU.
"""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle as O
from sspec_workload import cycle_state, make_workload, pack_rows
from tests.helpers import (assert_attn_close, assert_lse_close, bf16_tensor_to_f64, check_topk,
                           dump_to_rows, host_pages, request_kv, rows_to_dump, say, DUMP_TOL)

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def S():
    from sparse_self_speculative_amd import sspec
    return sspec


def _kv(S, w):
    return S.PagedKV(w.k_pages.to(DEV), w.v_pages.to(DEV), w.block_table.to(DEV))


def _run_verify(S, w, kv, lengths):
    n, hq, hkv, k = w.batch, w.num_q_heads, w.num_kv_heads, w.k
    max_ctx = int(w.caps.max())
    lstride = -(-max_ctx // 16) * 16
    q = w.qbank[:, : k + 1].contiguous().to(DEV)
    seq = torch.arange(n, dtype=torch.int32, device=DEV)
    ctx = torch.as_tensor(np.asarray(lengths), dtype=torch.int32, device=DEV)
    out = torch.empty_like(q)
    lse = torch.empty(n, k + 1, hq, dtype=torch.float32, device=DEV)
    mp = S.dump_pitch(hq, hkv, k)
    logits = torch.full((n, hkv, lstride // 16, mp, 16), float("nan"), dtype=torch.float32, device=DEV)
    ws = S.workspace(S.verify_workspace_size(n, max_ctx, hq, hkv, k))
    S.verify_attn(kv, q, seq, ctx, n, max_ctx, hq, k, w.sm_scale, out, lse, logits, lstride, ws)
    torch.cuda.synchronize()
    assert S.read_device_error(ws) == 0
    return q, seq, ctx, out, lse, logits, max_ctx, lstride


VERIFY_CASES = [
    # (hq, hkv, k, lengths)
    (16, 8, 8, [2048]),                       # the single-request workload shape
    (32, 8, 8, [37, 1500, 2100, 4097]),       # 3 query tiles, 1..5 splits, ragged tails
    (40, 8, 8, [1111, 2049]),                 # G = 5
    (8, 8, 0, [1, 16, 17, 1025]),             # single query, G = 1, L = 1
    (24, 8, 16, [300, 3000]),                 # G = 3, k = 16 -> 4 query tiles
    (16, 2, 3, [4, 999]),                     # G = 8
    (32, 8, 16, [2500]),                      # G*(k+1) = 68 -> 5 query tiles
    (16, 2, 8, [3000]),                       # G = 8, 72 rows in several split partials
]


@pytest.mark.parametrize("hq,hkv,k,lengths", VERIFY_CASES)
def test_verify_parity(S, hq, hkv, k, lengths):
    say(f"[verify] hq={hq} hkv={hkv} k={k} L={lengths}")
    w = make_workload(dict(hq=hq, hkv=hkv, k=k, s=0.05, batch=len(lengths)), seed=hq + k,
                      lengths=lengths)
    kv = _kv(S, w)
    q, seq, ctx, out, lse, logits, max_ctx, lstride = _run_verify(S, w, kv, lengths)
    kp, vp, bt = host_pages(w)
    q64 = bf16_tensor_to_f64(q)
    o64 = bf16_tensor_to_f64(out)
    lse_h, lg_h = lse.cpu().numpy(), logits.cpu().numpy()
    for r, L in enumerate(lengths):
        kc, vc = request_kv(kp, vp, bt, r, L)
        o_ref, lse_ref, lg_ref = O.verify_attention(q64[r], kc, vc, w.sm_scale)
        assert_attn_close(o64[r], o_ref, f"verify O r={r}")
        assert_lse_close(lse_h[r], lse_ref, f"verify LSE r={r}")
        got = dump_to_rows(lg_h[r], hq, hkv, k, L)
        fin = np.isfinite(lg_ref)
        assert np.array_equal(np.isfinite(got), fin), f"dump mask differs r={r}"
        assert np.abs(got[fin] - lg_ref[fin]).max() <= DUMP_TOL
        nb = -(-L // 16)
        last = lg_h[r][:, nb - 1, :, L - 16 * (nb - 1):]
        assert np.all(np.isneginf(last)), "dump keys past L must be -inf"
        G = hq // hkv
        assert np.all(np.isneginf(lg_h[r][:, :nb, G * (k + 1):, :])), "dump padding rows must be -inf"


def test_verify_large_logit_jump(S):
    """Keys in the middle of a chunk whose logits rise far (hundreds of natural
    log units) above the chunk's first page: the verify restarts its pass with
    a higher softmax reference; O, LSE and the dump must still match."""
    hq, hkv, k, lengths = 16, 8, 8, [1500, 3000]
    say(f"[verify jump] hq={hq} hkv={hkv} k={k} L={lengths}")
    w = make_workload(dict(hq=hq, hkv=hkv, k=k, s=0.05, batch=len(lengths)), seed=23, lengths=lengths)
    G = hq // hkv
    bt = w.block_table
    for r, pos in ((0, 700), (1, 2100)):
        for h in range(hkv):
            # aligned with the group's first query: a logit of ~8|q|^2/sqrt(d) ~ 90
            big = (8.0 * w.qbank[r, 0, h * G].float()).to(torch.bfloat16)
            for t in range(pos, pos + 16):
                phys = int(bt[r, t // 16])
                w.k_pages[phys, h, t % 16] = big.to(w.k_pages.device)
    kv = _kv(S, w)
    q, seq, ctx, out, lse, logits, max_ctx, lstride = _run_verify(S, w, kv, lengths)
    kp, vp, btn = host_pages(w)
    q64 = bf16_tensor_to_f64(q)
    o64 = bf16_tensor_to_f64(out)
    lse_h, lg_h = lse.cpu().numpy(), logits.cpu().numpy()
    for r, L in enumerate(lengths):
        kc, vc = request_kv(kp, vp, btn, r, L)
        o_ref, lse_ref, lg_ref = O.verify_attention(q64[r], kc, vc, w.sm_scale)
        fin = np.isfinite(lg_ref)
        assert lg_ref[fin].max() - lg_ref[:, :, :16][np.isfinite(lg_ref[:, :, :16])].max() > 64, "no jump planted"
        assert_attn_close(o64[r], o_ref, f"verify jump O r={r}")
        assert_lse_close(lse_h[r], lse_ref, f"verify jump LSE r={r}")
        got = dump_to_rows(lg_h[r], hq, hkv, k, L)
        assert np.array_equal(np.isfinite(got), fin), f"dump mask differs r={r}"
        rel = np.abs(got[fin] - lg_ref[fin]) / np.maximum(1.0, np.abs(lg_ref[fin]))
        assert rel.max() <= DUMP_TOL


TOPK_CASES = [
    (16, 8, 8, [2048], 0.05),
    (32, 8, 8, [37, 1500, 2100, 4097], 0.05),
    (32, 8, 4, [3000, 1200], 0.01),
    (16, 8, 8, [700, 2600], 1.0),
    (40, 8, 8, [5000], 0.1),
    (32, 8, 16, [3000, 1000, 77], 0.05),        # k = 16: 68 rows per group, 5 query tiles
    (8, 8, 8, [3000, 900], 0.1),                # G = 1: 9 rows, one load per page block
    (64, 8, 8, [2500, 1300], 0.05),             # G = 8: 72 rows, five loads per page block
]


@pytest.mark.parametrize("hq,hkv,k,lengths,s", TOPK_CASES)
def test_verify_then_topk_parity(S, hq, hkv, k, lengths, s):
    say(f"[topk] hq={hq} hkv={hkv} k={k} L={lengths} s={s}")
    w = make_workload(dict(hq=hq, hkv=hkv, k=k, s=s, batch=len(lengths)), seed=7 + k,
                      lengths=lengths)
    kv = _kv(S, w)
    q, seq, ctx, out, lse, logits, max_ctx, lstride = _run_verify(S, w, kv, lengths)
    n = w.batch
    sel_stride = O.select_count(max_ctx, s)
    sel = torch.full((n, hkv, sel_stride), -7, dtype=torch.int32, device=DEV)
    cnt = torch.zeros(n, dtype=torch.int32, device=DEV)
    sl = torch.zeros(n, dtype=torch.int32, device=DEV)
    ws = S.workspace(S.pillar_topk_workspace_size(n, max_ctx, hkv))
    S.pillar_topk(logits, lse, lstride, seq, ctx, n, n, max_ctx, hq, hkv, k, s, sel, sel_stride,
                  cnt, sl, ws)
    torch.cuda.synchronize()
    assert S.read_device_error(ws) == 0
    kp, vp, bt = host_pages(w)
    q64 = bf16_tensor_to_f64(q)
    sel_h, cnt_h, sl_h = sel.cpu().numpy(), cnt.cpu().numpy(), sl.cpu().numpy()
    ndiff = 0
    for r, L in enumerate(lengths):
        kc, vc = request_kv(kp, vp, bt, r, L)
        _, lse_ref, lg_ref = O.verify_attention(q64[r], kc, vc, w.sm_scale)
        S_ref = O.pillar_scores(lg_ref, lse_ref, hkv)
        sel_ref, K = O.pillar_topk(lg_ref, lse_ref, hkv, s)
        assert cnt_h[r] == K and sl_h[r] == L
        for h in range(hkv):
            ndiff += check_topk(sel_h[r, h], int(cnt_h[r]), S_ref[h], sel_ref[h], f"r={r} h={h}")
    say(f"   near-tie differences: {ndiff}")


def test_topk_from_oracle_dump(S):
    """Selection alone, fed with the oracle's own dump (rounded to fp32)."""
    say("[topk-oracle-dump]")
    rng = np.random.default_rng(3)
    hq, hkv, k, L, d = 16, 4, 5, 3001, 128
    G = hq // hkv
    q = rng.standard_normal((k + 1, hq, d))
    kc = rng.standard_normal((hkv, L, d))
    vc = rng.standard_normal((hkv, L, d))
    _, lse_ref, lg_ref = O.verify_attention(q, kc, vc, 1 / math.sqrt(d))
    lstride = -(-L // 16) * 16
    lg = rows_to_dump(lg_ref.astype(np.float32), hkv, k, lstride, S.dump_pitch(hq, hkv, k))[None]
    logits = torch.from_numpy(lg).to(DEV)
    lse = torch.from_numpy(lse_ref[None].astype(np.float32)).to(DEV)
    seq = torch.zeros(1, dtype=torch.int32, device=DEV)
    ctx = torch.tensor([L], dtype=torch.int32, device=DEV)
    s = 0.05
    K = O.select_count(L, s)
    sel = torch.zeros(1, hkv, K, dtype=torch.int32, device=DEV)
    cnt = torch.zeros(1, dtype=torch.int32, device=DEV)
    sl = torch.zeros(1, dtype=torch.int32, device=DEV)
    ws = S.workspace(S.pillar_topk_workspace_size(1, L, hkv))
    S.pillar_topk(logits, lse, lstride, seq, ctx, 1, 1, L, hq, hkv, k, s, sel, K, cnt, sl, ws)
    torch.cuda.synchronize()
    S_ref = O.pillar_scores(lg_ref, lse_ref, hkv)
    sel_ref, _ = O.pillar_topk(lg_ref, lse_ref, hkv, s)
    for h in range(hkv):
        check_topk(sel.cpu().numpy()[0, h], int(cnt.cpu()[0]), S_ref[h], sel_ref[h], f"h={h}")
    assert G == 4


DRAFT_CASES = [
    # (hq, hkv, lengths(sel_len), extra (ctx - sel_len), s)
    (16, 8, [2048], [1], 0.05),
    (32, 8, [1500, 4097, 300], [3, 8, 1], 0.05),
    (32, 8, [2100, 900], [-5, 0], 0.05),        # rollback / no tail
    (40, 8, [4100], [2], 1.0),                   # s = 1: full attention, many splits
    (8, 8, [20, 50], [4, 0], 0.3),
    (16, 2, [777], [5], 0.1),                    # G = 8
    (16, 2, [6000], [3], 0.2),                   # G = 8, several split partials
    (8, 8, [5000], [2], 0.25),                   # G = 1, several split partials
]


@pytest.mark.parametrize("hq,hkv,lengths,extra,s", DRAFT_CASES)
def test_draft_parity(S, hq, hkv, lengths, extra, s):
    say(f"[draft] hq={hq} hkv={hkv} L={lengths} extra={extra} s={s}")
    k = 8
    w = make_workload(dict(hq=hq, hkv=hkv, k=k, s=s, batch=len(lengths)), seed=11 + hq,
                      lengths=lengths)
    kp, vp, bt = host_pages(w)
    n = w.batch
    max_ctx = int(w.caps.max())
    sel_stride = O.select_count(max_ctx, s)
    sel_np = np.zeros((n, hkv, sel_stride), np.int32)
    cnt_np = np.zeros(n, np.int32)
    sl_np = np.asarray(lengths, np.int32)
    q64v = bf16_tensor_to_f64(w.qbank)
    sels = []
    for r, L in enumerate(lengths):
        kc, vc = request_kv(kp, vp, bt, r, L)
        _, lse_ref, lg_ref = O.verify_attention(q64v[r, : k + 1], kc, vc, w.sm_scale)
        sel_ref, K = O.pillar_topk(lg_ref, lse_ref, hkv, s)
        sel_np[r, :, :K] = sel_ref
        cnt_np[r] = K
        sels.append(sel_ref)
    ctx_np = np.asarray([L + e for L, e in zip(lengths, extra)], np.int32)
    qd = torch.stack([w.qbank[r, k + max(1, min(k, e))] for r, e in enumerate(extra)]).contiguous()
    kv = _kv(S, w)
    out = torch.empty_like(qd, device=DEV)
    lse = torch.empty(n, hq, dtype=torch.float32, device=DEV)
    ws = S.workspace(S.draft_workspace_size(n, max_ctx, hq, hkv))
    S.sparse_draft_attn(kv, qd.to(DEV), torch.arange(n, dtype=torch.int32, device=DEV),
                        torch.from_numpy(ctx_np).to(DEV), torch.from_numpy(sel_np).to(DEV),
                        sel_stride, torch.from_numpy(cnt_np).to(DEV),
                        torch.from_numpy(sl_np).to(DEV), n, max_ctx, hq, w.sm_scale, out, lse, ws)
    torch.cuda.synchronize()
    assert S.read_device_error(ws) == 0
    o64 = bf16_tensor_to_f64(out)
    q64 = bf16_tensor_to_f64(qd)
    lse_h = lse.cpu().numpy()
    for r in range(n):
        c = int(ctx_np[r])
        kc, vc = request_kv(kp, vp, bt, r, max(c, lengths[r]))
        o_ref, l_ref = O.sparse_draft_attention(q64[r], kc, vc, sels[r], lengths[r], c, w.sm_scale)
        assert_attn_close(o64[r], o_ref, f"draft O r={r}")
        assert_lse_close(lse_h[r], l_ref, f"draft LSE r={r}")


def _oracle_selection_state(w, kp, vp, bt):
    """Selections every request would hold after verifying at its L."""
    k, hkv, s = w.k, w.num_kv_heads, w.s
    q64 = bf16_tensor_to_f64(w.qbank)
    sels = []
    for r in range(w.batch):
        L = int(w.verify_lens[r])
        kc, vc = request_kv(kp, vp, bt, r, L)
        _, lse_ref, lg_ref = O.verify_attention(q64[r, : k + 1], kc, vc, w.sm_scale)
        sel_ref, _ = O.pillar_topk(lg_ref, lse_ref, hkv, s)
        sels.append(sel_ref)
    return sels


UNIFIED_CASES = [
    # (hq, hkv, k, s, lengths)
    (32, 8, 8, 0.05, [1200, 2600, 333, 4100, 1800, 950, 2222, 1500, 3000, 64, 2048, 1700]),
    (16, 8, 4, 0.1, [500, 1030, 2047, 33, 800, 1600, 700]),
    (40, 8, 8, 0.05, [1500, 2900, 1000, 2000, 2500, 1200, 600, 3100, 1800, 900]),
    # k = 16 (G = 4: 68 rows, the 5-query-tile instance), more buckets than requests
    (32, 8, 16, 0.05, [1500, 2900, 1000, 2000, 2500, 1200, 600, 3100, 1800, 900, 4200, 700]),
    (32, 8, 4, 0.01, [3000, 5200, 1000, 2400, 4100, 800]),          # s = 0.01
    (32, 8, 8, 1.0, [1200, 2600, 333, 1800, 950, 2222, 1500, 640, 3000, 1100]),   # s = 1: full attention
    # rows of 4 to 6 score chunks (2048 keys each)
    (32, 8, 4, 0.05, [8200, 9000, 1200, 12000, 600, 3000]),
    # G = 8 (72 rows: the 5-query-tile instance, verify and draft split partials of 72 and 8 rows)
    (64, 8, 8, 0.05, [1500, 3000, 800, 2200, 4100, 600, 1900, 2700, 1200, 5000]),
    # G = 1 (9 rows in one tile; draft partials of one row)
    (8, 8, 8, 0.25, [1500, 3000, 800, 2200, 4100, 600, 1900, 2700, 1200, 5000]),
]


@pytest.mark.parametrize("hq,hkv,k,s,lengths", UNIFIED_CASES)
def test_unified_parity(S, hq, hkv, k, s, lengths):
    say(f"[unified] hq={hq} hkv={hkv} k={k} s={s} B={len(lengths)}")
    w = make_workload(dict(hq=hq, hkv=hkv, k=k, s=s, batch=len(lengths)), seed=5 + hq,
                      lengths=lengths)
    kp, vp, bt = host_pages(w)
    B = w.batch
    sels0 = _oracle_selection_state(w, kp, vp, bt)
    max_ctx = int(w.caps.max())
    sel_stride = O.select_count(max_ctx, s)
    max_verify = int(np.bincount(w.bucket_ids).max())
    kv = _kv(S, w)
    ws = S.workspace(S.unified_workspace_size(B, max_verify, max_ctx, hq, hkv, k))
    for t in [0, 1, k]:
        vb, isv, ctx, step = cycle_state(w, t)
        say(f"   launch t={t} verify_bucket={vb} n_verify={int(isv.sum())}")
        sel_np = np.zeros((B, hkv, sel_stride), np.int32)
        for r in range(B):
            sel_np[r, :, : sels0[r].shape[1]] = sels0[r]
        cnt_np = np.array([sels0[r].shape[1] for r in range(B)], np.int32)
        sl_np = w.verify_lens.astype(np.int32)
        sel_t, cnt_t, sl_t = (torch.from_numpy(a).to(DEV) for a in (sel_np, cnt_np, sl_np))
        q = pack_rows(w, isv, step, DEV)
        out = torch.empty_like(q)
        lse = torch.empty(q.shape[0], hq, dtype=torch.float32, device=DEV)
        S.unified_attn(kv, q, torch.from_numpy(ctx.astype(np.int32)).to(DEV),
                       torch.from_numpy(w.bucket_ids).to(DEV), vb, B, max_verify, max_ctx, hq, k,
                       s, w.sm_scale, sel_t, sel_stride, cnt_t, sl_t, out, lse, ws)
        torch.cuda.synchronize()
        assert S.read_device_error(ws) == 0
        o_ref, l_ref, sel_ref, sl_ref = O.unified_step(
            bf16_tensor_to_f64(q), kp, vp, bt, ctx, isv, k, s, w.sm_scale, sels0, sl_np)
        assert_attn_close(bf16_tensor_to_f64(out), o_ref, f"unified O t={t}")
        assert_lse_close(lse.cpu().numpy(), l_ref, f"unified LSE t={t}")
        sel_h, cnt_h, sl_h = sel_t.cpu().numpy(), cnt_t.cpu().numpy(), sl_t.cpu().numpy()
        assert np.array_equal(sl_h, sl_ref)
        for r in np.nonzero(isv)[0]:
            L = int(ctx[r])
            kc, vc = request_kv(kp, vp, bt, r, L)
            nr = np.where(isv, k + 1, 1)
            off = int(np.concatenate([[0], np.cumsum(nr)])[r])
            _, lse_r, lg_r = O.verify_attention(bf16_tensor_to_f64(q)[off: off + k + 1], kc, vc,
                                                w.sm_scale)
            S_ref = O.pillar_scores(lg_r, lse_r, hkv)
            for h in range(hkv):
                check_topk(sel_h[r, h], int(cnt_h[r]), S_ref[h], sel_ref[r][h], f"t={t} r={r} h={h}")
        for r in np.nonzero(~isv)[0]:
            assert cnt_h[r] == cnt_np[r] and np.array_equal(sel_h[r], sel_np[r])


def test_unified_matches_separate_launches(S):
    """The persistent launch and the three separate entry points agree."""
    say("[unified-vs-separate]")
    hq, hkv, k, s = 32, 8, 8, 0.05
    lengths = [1300, 2500, 900, 3300, 1700, 2100, 600, 1900, 2800, 1100]
    w = make_workload(dict(hq=hq, hkv=hkv, k=k, s=s, batch=len(lengths)), seed=99, lengths=lengths)
    kv = _kv(S, w)
    B = w.batch
    max_ctx = int(w.caps.max())
    sel_stride = O.select_count(max_ctx, s)
    vb, isv, ctx, step = cycle_state(w, 2)
    ctx_t = torch.from_numpy(ctx.astype(np.int32)).to(DEV)
    # selections for the drafting requests: any valid ascending sets
    rng = np.random.default_rng(1)
    sel_np = np.zeros((B, hkv, sel_stride), np.int32)
    cnt_np = np.zeros(B, np.int32)
    for r in range(B):
        L = int(w.verify_lens[r])
        K = O.select_count(L, s)
        cnt_np[r] = K
        for h in range(hkv):
            sel_np[r, h, :K] = np.sort(rng.choice(L, K, replace=False))
    sl_np = w.verify_lens.astype(np.int32)
    q = pack_rows(w, isv, step, DEV)
    # unified
    sel_u, cnt_u, sl_u = (torch.from_numpy(a.copy()).to(DEV) for a in (sel_np, cnt_np, sl_np))
    out_u = torch.empty_like(q)
    lse_u = torch.empty(q.shape[0], hq, dtype=torch.float32, device=DEV)
    mv = int(isv.sum())
    wsu = S.workspace(S.unified_workspace_size(B, mv, max_ctx, hq, hkv, k))
    S.unified_attn(kv, q, ctx_t, torch.from_numpy(w.bucket_ids).to(DEV), vb, B, mv, max_ctx, hq, k,
                   s, w.sm_scale, sel_u, sel_stride, cnt_u, sl_u, out_u, lse_u, wsu)
    # separate
    nr = np.where(isv, k + 1, 1)
    off = np.concatenate([[0], np.cumsum(nr)])
    vid = np.nonzero(isv)[0]
    did = np.nonzero(~isv)[0]
    qv = torch.stack([q[off[r]: off[r] + k + 1] for r in vid]).contiguous()
    qd = torch.stack([q[off[r]] for r in did]).contiguous()
    nv, nd = len(vid), len(did)
    lstride = -(-max_ctx // 16) * 16
    out_v = torch.empty_like(qv)
    lse_v = torch.empty(nv, k + 1, hq, dtype=torch.float32, device=DEV)
    logits = torch.empty(nv, hkv, lstride // 16, S.dump_pitch(hq, hkv, k), 16, dtype=torch.float32, device=DEV)
    seq_v = torch.from_numpy(vid.astype(np.int32)).to(DEV)
    seq_d = torch.from_numpy(did.astype(np.int32)).to(DEV)
    wsv = S.workspace(S.verify_workspace_size(nv, max_ctx, hq, hkv, k))
    S.verify_attn(kv, qv, seq_v, ctx_t, nv, max_ctx, hq, k, w.sm_scale, out_v, lse_v, logits,
                  lstride, wsv)
    sel_s, cnt_s, sl_s = (torch.from_numpy(a.copy()).to(DEV) for a in (sel_np, cnt_np, sl_np))
    wst = S.workspace(S.pillar_topk_workspace_size(nv, max_ctx, hkv))
    S.pillar_topk(logits, lse_v, lstride, seq_v, ctx_t, nv, B, max_ctx, hq, hkv, k, s, sel_s,
                  sel_stride, cnt_s, sl_s, wst)
    out_d = torch.empty_like(qd)
    lse_d = torch.empty(nd, hq, dtype=torch.float32, device=DEV)
    wsd = S.workspace(S.draft_workspace_size(nd, max_ctx, hq, hkv))
    sel_d, cnt_d, sl_d = (torch.from_numpy(a.copy()).to(DEV) for a in (sel_np, cnt_np, sl_np))
    S.sparse_draft_attn(kv, qd, seq_d, ctx_t, sel_d, sel_stride, cnt_d, sl_d, nd, max_ctx, hq,
                        w.sm_scale, out_d, lse_d, wsd)
    torch.cuda.synchronize()
    for i, r in enumerate(vid):
        assert torch.equal(out_u[off[r]: off[r] + k + 1].view(torch.int16), out_v[i].view(torch.int16))
        assert torch.equal(lse_u[off[r]: off[r] + k + 1], lse_v[i])
    for i, r in enumerate(did):
        assert torch.equal(out_u[off[r]].view(torch.int16), out_d[i].view(torch.int16))
        assert torch.equal(lse_u[off[r]], lse_d[i])
    assert torch.equal(sel_u, sel_s) and torch.equal(cnt_u, cnt_s) and torch.equal(sl_u, sl_s)
    for ws in (wsu, wsv, wst, wsd):
        assert S.read_device_error(ws) == 0


def test_unified_deterministic_and_reusable(S):
    """Two launches on the same workspace give bit-identical results."""
    say("[unified-repeat]")
    hq, hkv, k, s = 32, 8, 8, 0.05
    lengths = [1000 + 137 * i for i in range(18)]
    w = make_workload(dict(hq=hq, hkv=hkv, k=k, s=s, batch=len(lengths)), seed=4, lengths=lengths)
    kv = _kv(S, w)
    B = w.batch
    max_ctx = int(w.caps.max())
    sel_stride = O.select_count(max_ctx, s)
    mv = int(np.bincount(w.bucket_ids).max())
    ws = S.workspace(S.unified_workspace_size(B, mv, max_ctx, hq, hkv, k))
    res = []
    for rep in range(3):
        vb, isv, ctx, step = cycle_state(w, 3)
        sel = torch.zeros(B, hkv, sel_stride, dtype=torch.int32, device=DEV)
        cnt = torch.zeros(B, dtype=torch.int32, device=DEV)
        sl = torch.from_numpy(w.verify_lens.astype(np.int32)).to(DEV)
        q = pack_rows(w, isv, step, DEV)
        out = torch.empty_like(q)
        lse = torch.empty(q.shape[0], hq, dtype=torch.float32, device=DEV)
        S.unified_attn(kv, q, torch.from_numpy(ctx.astype(np.int32)).to(DEV),
                       torch.from_numpy(w.bucket_ids).to(DEV), vb, B, mv, max_ctx, hq, k, s,
                       w.sm_scale, sel, sel_stride, cnt, sl, out, lse, ws)
        torch.cuda.synchronize()
        res.append((out.clone(), lse.clone(), sel.clone()))
    assert S.read_device_error(ws) == 0
    for o, l, se in res[1:]:
        assert torch.equal(o.view(torch.int16), res[0][0].view(torch.int16))
        assert torch.equal(l, res[0][1]) and torch.equal(se, res[0][2])


def test_unified_full_size_sampled(S):
    """The benchmark's own workload and launch sequence (Qwen3-8B attention
    shape, batch 128, contexts lognormal mean 12K up to 32K, k = 8, s = 0.05,
    seed 2): after the set-up cycle, one more launch is checked on a sample
    the oracle computes one request at a time: the O, LSE and Top-K of the
    longest and one other verifying request, and the O and LSE of six
    drafting requests (against the selections the GPU holds going in)."""
    from sspec_workload import to_numpy_bf16, workload_spec
    say("[unified full size] qwen3-8b shape B=128 seed 2")
    w = make_workload(workload_spec(2), seed=2, device=DEV)
    B, hq, hkv, k, s = w.batch, w.num_q_heads, w.num_kv_heads, w.k, w.s
    kp1 = k + 1
    max_ctx = int(w.caps.max())
    sel_stride = math.ceil(s * max_ctx)
    max_verify = int(np.bincount(w.bucket_ids, minlength=kp1).max())
    kv = _kv(S, w)
    ws = S.workspace(S.unified_workspace_size(B, max_verify, max_ctx, hq, hkv, k))
    sel = torch.zeros(B, hkv, sel_stride, dtype=torch.int32, device=DEV)
    cnt = torch.zeros(B, dtype=torch.int32, device=DEV)
    sl = torch.from_numpy(w.verify_lens.astype(np.int32)).to(DEV)
    bk = torch.from_numpy(w.bucket_ids).to(DEV)

    def launch(t):
        vb, isv, ctx, step = cycle_state(w, t)
        q = pack_rows(w, isv, step, DEV)
        out = torch.empty_like(q)
        lse = torch.empty(q.shape[0], hq, dtype=torch.float32, device=DEV)
        S.unified_attn(kv, q, torch.from_numpy(ctx.astype(np.int32)).to(DEV), bk, vb, B, max_verify,
                       max_ctx, hq, k, s, w.sm_scale, sel, sel_stride, cnt, sl, out, lse, ws)
        return q, out, lse, isv, ctx

    for t in range(kp1):   # set-up cycle: every request verifies once
        launch(t)
    torch.cuda.synchronize()
    assert S.read_device_error(ws) == 0
    sel_in, cnt_in, sl_in = sel.cpu().numpy(), cnt.cpu().numpy(), sl.cpu().numpy()
    t = kp1 + 3
    say(f"   checked launch t={t}")
    q, out, lse, isv, ctx = launch(t)
    torch.cuda.synchronize()
    assert S.read_device_error(ws) == 0
    q64, o64, lse_h = bf16_tensor_to_f64(q), bf16_tensor_to_f64(out), lse.cpu().numpy()
    sel_h, cnt_h, sl_h = sel.cpu().numpy(), cnt.cpu().numpy(), sl.cpu().numpy()
    off = np.concatenate([[0], np.cumsum(np.where(isv, kp1, 1))])

    def kv_of(r, n):   # float64 K, V of request r's first n tokens, from its own pages only
        pages = w.block_table[r, : -(-n // 16)].to(DEV).long()
        kp = to_numpy_bf16(w.k_pages[pages])
        vp = to_numpy_bf16(w.v_pages[pages])
        row = np.arange(pages.shape[0])
        return O.gather_kv(kp, row, n, 16), O.gather_kv(vp, row, n, 16)

    rng = np.random.default_rng(0)
    vid = np.nonzero(isv)[0]
    for r in {int(vid[np.argmax(ctx[vid])]), int(rng.choice(vid))}:
        L = int(ctx[r])
        say(f"   verify r={r} L={L}")
        kc, vc = kv_of(r, L)
        o_ref, lse_ref, lg_ref = O.verify_attention(q64[off[r]: off[r] + kp1], kc, vc, w.sm_scale)
        assert_attn_close(o64[off[r]: off[r] + kp1], o_ref, f"full-size verify O r={r}")
        assert_lse_close(lse_h[off[r]: off[r] + kp1], lse_ref, f"full-size verify LSE r={r}")
        S_ref = O.pillar_scores(lg_ref, lse_ref, hkv)
        sel_ref, _ = O.pillar_topk(lg_ref, lse_ref, hkv, s)
        assert sl_h[r] == L
        for h in range(hkv):
            check_topk(sel_h[r, h], int(cnt_h[r]), S_ref[h], sel_ref[h], f"full-size r={r} h={h}")
    did = np.nonzero(~isv)[0]
    for r in rng.choice(did, 6, replace=False):
        r = int(r)
        L = int(ctx[r])
        kc, vc = kv_of(r, L)
        sets = [sel_in[r, h, : cnt_in[r]] for h in range(hkv)]
        o_ref, lse_ref = O.sparse_draft_attention(q64[off[r]], kc, vc, sets, int(sl_in[r]), L, w.sm_scale)
        assert_attn_close(o64[off[r]][None], o_ref[None], f"full-size draft O r={r}")
        assert_lse_close(lse_h[off[r]][None], lse_ref[None], f"full-size draft LSE r={r}")
        assert cnt_h[r] == cnt_in[r] and np.array_equal(sel_h[r], sel_in[r])


def test_verify_empty_and_error_paths(S):
    """n = 0 does nothing; arguments the host rejects raise before any launch;
    a request whose context exceeds max_ctx, or whose block table points
    outside the pool, raises its device error bit (the kernel's own range
    checks: the first is skipped, the second reads page 0 instead) while the
    other requests of the launch stay exact."""
    say("[verify edge] empty batch, bad stride, bad ctx, bad page")
    hq, hkv, k, lengths = 16, 8, 8, [700, 1500, 900]
    w = make_workload(dict(hq=hq, hkv=hkv, k=k, s=0.05, batch=len(lengths)), seed=31, lengths=lengths)
    kv = _kv(S, w)
    n = w.batch
    max_ctx = int(w.caps.max())
    lstride = -(-max_ctx // 16) * 16
    q = w.qbank[:, : k + 1].contiguous().to(DEV)
    seq = torch.arange(n, dtype=torch.int32, device=DEV)
    out = torch.full_like(q, 7)
    lse = torch.full((n, k + 1, hq), 7.0, dtype=torch.float32, device=DEV)
    logits = torch.empty(n, hkv, lstride // 16, S.dump_pitch(hq, hkv, k), 16, dtype=torch.float32, device=DEV)
    ws = S.workspace(S.verify_workspace_size(n, max_ctx, hq, hkv, k))
    ctx = torch.as_tensor(np.asarray(lengths), dtype=torch.int32, device=DEV)
    # empty batch: nothing launched, nothing written
    S.verify_attn(kv, q, seq, ctx, 0, max_ctx, hq, k, w.sm_scale, out, lse, logits, lstride, ws)
    torch.cuda.synchronize()
    assert bool((lse == 7.0).all()) and S.read_device_error(ws) == 0
    # host-side rejection: logit_stride not a multiple of 16
    with pytest.raises(S.SspecError):
        S.verify_attn(kv, q, seq, ctx, n, max_ctx, hq, k, w.sm_scale, out, lse, logits, lstride + 1, ws)
    # request 1 past max_ctx: skipped with SSPEC_DEV_ERR_CTX_RANGE
    ctx_bad = torch.as_tensor(np.asarray([lengths[0], max_ctx + 1, lengths[2]]), dtype=torch.int32, device=DEV)
    S.verify_attn(kv, q, seq, ctx_bad, n, max_ctx, hq, k, w.sm_scale, out, lse, logits, lstride, ws)
    torch.cuda.synchronize()
    assert S.read_device_error(ws) & S.DEV_ERR["CTX_RANGE"]
    assert bool((lse[1] == 7.0).all()), "the skipped request must stay untouched"
    kp, vp, bt = host_pages(w)
    q64 = bf16_tensor_to_f64(q)
    for r in (0, 2):
        kc, vc = request_kv(kp, vp, bt, r, lengths[r])
        o_ref, lse_ref, _ = O.verify_attention(q64[r], kc, vc, w.sm_scale)
        assert_attn_close(bf16_tensor_to_f64(out)[r], o_ref, f"bad-ctx neighbour O r={r}")
        assert_lse_close(lse.cpu().numpy()[r], lse_ref, f"bad-ctx neighbour LSE r={r}")
    # request 2's first block-table entry outside the pool: SSPEC_DEV_ERR_PAGE_RANGE
    bt_bad = w.block_table.clone().to(DEV)
    bt_bad[2, 0] = w.k_pages.shape[0] + 5
    kv_bad = S.PagedKV(w.k_pages.to(DEV), w.v_pages.to(DEV), bt_bad)
    S.verify_attn(kv_bad, q, seq, ctx, n, max_ctx, hq, k, w.sm_scale, out, lse, logits, lstride, ws)
    torch.cuda.synchronize()
    assert S.read_device_error(ws) & S.DEV_ERR["PAGE_RANGE"]
    for r in (0, 1):
        kc, vc = request_kv(kp, vp, bt, r, lengths[r])
        o_ref, lse_ref, _ = O.verify_attention(q64[r], kc, vc, w.sm_scale)
        assert_attn_close(bf16_tensor_to_f64(out)[r], o_ref, f"bad-page neighbour O r={r}")


def test_unified_too_many_verify_flags_and_skips(S):
    """A unified launch whose verify bucket holds more requests than the
    max_verify it was sized for: the requests past the limit are skipped with
    SSPEC_DEV_ERR_TOO_MANY_VERIFY (outputs untouched, selections unchanged),
    the others are computed as usual."""
    say("[unified edge] more verify requests than max_verify")
    hq, hkv, k, s = 16, 8, 4, 0.1
    lengths = [500, 1030, 2047, 800, 1600, 700, 900]
    w = make_workload(dict(hq=hq, hkv=hkv, k=k, s=s, batch=len(lengths)), seed=41, lengths=lengths)
    kp, vp, bt = host_pages(w)
    B = w.batch
    sels0 = _oracle_selection_state(w, kp, vp, bt)
    max_ctx = int(w.caps.max())
    sel_stride = O.select_count(max_ctx, s)
    vb, isv, ctx, step = cycle_state(w, 0)
    nv = int(isv.sum())
    if nv < 2:
        pytest.skip("the seeded bucket assignment put fewer than 2 requests in bucket 0")
    max_verify = nv - 1
    kv = _kv(S, w)
    ws = S.workspace(S.unified_workspace_size(B, max_verify, max_ctx, hq, hkv, k))
    sel_np = np.zeros((B, hkv, sel_stride), np.int32)
    for r in range(B):
        sel_np[r, :, : sels0[r].shape[1]] = sels0[r]
    cnt_np = np.array([sels0[r].shape[1] for r in range(B)], np.int32)
    sl_np = w.verify_lens.astype(np.int32)
    sel_t, cnt_t, sl_t = (torch.from_numpy(a.copy()).to(DEV) for a in (sel_np, cnt_np, sl_np))
    q = pack_rows(w, isv, step, DEV)
    out = torch.full_like(q, 7)
    lse = torch.full((q.shape[0], hq), 7.0, dtype=torch.float32, device=DEV)
    S.unified_attn(kv, q, torch.from_numpy(ctx.astype(np.int32)).to(DEV), torch.from_numpy(w.bucket_ids).to(DEV),
                   vb, B, max_verify, max_ctx, hq, k, s, w.sm_scale, sel_t, sel_stride, cnt_t, sl_t, out, lse, ws)
    torch.cuda.synchronize()
    assert S.read_device_error(ws) & S.DEV_ERR["TOO_MANY_VERIFY"]
    vid = np.nonzero(isv)[0]
    skipped = int(vid[-1])   # verify requests are counted in request order
    off = np.concatenate([[0], np.cumsum(np.where(isv, k + 1, 1))])
    lse_h, sel_h = lse.cpu().numpy(), sel_t.cpu().numpy()
    assert np.all(lse_h[off[skipped]: off[skipped] + k + 1] == 7.0)
    assert np.array_equal(sel_h[skipped], sel_np[skipped])
    o_ref, l_ref, _, _ = O.unified_step(bf16_tensor_to_f64(q), kp, vp, bt, ctx, isv, k, s, w.sm_scale, sels0, sl_np)
    o64 = bf16_tensor_to_f64(out)
    for r in range(B):
        if r == skipped:
            continue
        rows = slice(off[r], off[r + 1])
        assert_attn_close(o64[rows], o_ref[rows], f"too-many-verify neighbour O r={r}")
        assert_lse_close(lse_h[rows], l_ref[rows], f"too-many-verify neighbour LSE r={r}")

"""Edge cases, error paths and robustness of the HIP path, through the C ABI.

  * one workspace shared by every entry point in turn, and a verify call of
    more than 512 requests made twice on one workspace: results identical to
    fresh-workspace calls and to the oracle;
  * a non-finite physical page 0 (the row masked draft positions read) does
    not reach any output;
  * each device error bit (short verify context, request id out of range,
    selected index out of range, too many selected entries) flags while the
    neighbouring requests stay exact; an empty draft set gives O = 0 and
    LSE = -inf; a unified launch with no verifying request;
  * a unified launch while torch GEMMs run on a second stream (its
    work-groups are then not all resident at once) gives the same bits;
  * each of the three Top-K paths (single pass, threshold-bin collection,
    two global passes) provably runs and agrees with the oracle.
Every case prints its name before touching the GPU.
"""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle as O
from sspec_workload import cycle_state, make_workload, pack_rows
from tests.helpers import (assert_attn_close, assert_lse_close, bf16_tensor_to_f64, check_topk,
                           expected_path, host_pages, request_kv, rows_to_dump, say, selection_paths)

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def S():
    from sparse_self_speculative_amd import sspec
    return sspec


def _kv(S, w, bt=None):
    return S.PagedKV(w.k_pages.to(DEV), w.v_pages.to(DEV), (w.block_table if bt is None else bt).to(DEV))


def _oracle_sels(w, kp, vp, bt):
    k, hkv, s = w.k, w.num_kv_heads, w.s
    q64 = bf16_tensor_to_f64(w.qbank)
    out = []
    for r in range(w.batch):
        L = int(w.verify_lens[r])
        kc, vc = request_kv(kp, vp, bt, r, L)
        _, lse, lg = O.verify_attention(q64[r, : k + 1], kc, vc, w.sm_scale)
        out.append(O.pillar_topk(lg, lse, hkv, s)[0])
    return out


def _sel_arrays(sels, B, hkv, stride):
    sel = np.zeros((B, hkv, stride), np.int32)
    for r in range(B):
        sel[r, :, : sels[r].shape[1]] = sels[r]
    cnt = np.array([x.shape[1] for x in sels], np.int32)
    return sel, cnt


def _dev(*arrs):
    return [torch.from_numpy(np.ascontiguousarray(a)).to(DEV) for a in arrs]


# --------------------------------------------------------- shared workspace
def test_workspace_shared_by_every_entry_point(S):
    """verify -> pillar_topk -> sparse_draft -> unified -> verify -> unified on
    ONE workspace (sized for the largest of them): every result is bitwise
    the result of the same call on a fresh workspace, and the unified launch
    matches the oracle.  (The entry points carve the workspace differently;
    each call's zero-state region must start clean.)"""
    say("[ws shared] verify -> topk -> draft -> unified -> verify -> unified")
    hq, hkv, k, s = 32, 8, 8, 0.05
    lengths = [1300, 2500, 900, 3300, 1700, 2100, 600, 1900, 2800, 1100, 2400, 1500]
    w = make_workload(dict(hq=hq, hkv=hkv, k=k, s=s, batch=len(lengths)), seed=61, lengths=lengths)
    kp, vp, bt = host_pages(w)
    kv = _kv(S, w)
    B = w.batch
    max_ctx = int(w.caps.max())
    sel_stride = O.select_count(max_ctx, s)
    sels0 = _oracle_sels(w, kp, vp, bt)
    sel_np, cnt_np = _sel_arrays(sels0, B, hkv, sel_stride)
    sl_np = w.verify_lens.astype(np.int32)
    vb, isv, ctx, step = cycle_state(w, 2)
    ctx_t = torch.from_numpy(ctx.astype(np.int32)).to(DEV)
    bk = torch.from_numpy(w.bucket_ids).to(DEV)
    q = pack_rows(w, isv, step, DEV)
    off = np.concatenate([[0], np.cumsum(np.where(isv, k + 1, 1))])
    vid, did = np.nonzero(isv)[0], np.nonzero(~isv)[0]
    nv, nd = len(vid), len(did)
    assert nv >= 1
    qv = torch.stack([q[off[r]: off[r] + k + 1] for r in vid]).contiguous()
    qd = torch.stack([q[off[r]] for r in did]).contiguous()
    seq_v = torch.from_numpy(vid.astype(np.int32)).to(DEV)
    seq_d = torch.from_numpy(did.astype(np.int32)).to(DEV)
    lstride = -(-max_ctx // 16) * 16
    mv = int(np.bincount(w.bucket_ids).max())
    sizes = dict(unified=S.unified_workspace_size(B, mv, max_ctx, hq, hkv, k),
                 verify=S.verify_workspace_size(nv, max_ctx, hq, hkv, k),
                 topk=S.pillar_topk_workspace_size(nv, max_ctx, hkv),
                 draft=S.draft_workspace_size(nd, max_ctx, hq, hkv))

    def do_verify(ws):
        out = torch.empty_like(qv)
        lse = torch.empty(nv, k + 1, hq, dtype=torch.float32, device=DEV)
        # blocks past a request's context are left untouched: start from zeros
        lg = torch.zeros(nv, hkv, lstride // 16, S.dump_pitch(hq, hkv, k), 16, dtype=torch.float32, device=DEV)
        S.verify_attn(kv, qv, seq_v, ctx_t, nv, max_ctx, hq, k, w.sm_scale, out, lse, lg, lstride, ws)
        return out, lse, lg

    def do_topk(ws, lg, lse):
        sel, cnt, sl = _dev(sel_np, cnt_np, sl_np)
        S.pillar_topk(lg, lse, lstride, seq_v, ctx_t, nv, B, max_ctx, hq, hkv, k, s, sel, sel_stride, cnt, sl, ws)
        return sel, cnt, sl

    def do_draft(ws):
        sel, cnt, sl = _dev(sel_np, cnt_np, sl_np)
        out = torch.empty_like(qd)
        lse = torch.empty(nd, hq, dtype=torch.float32, device=DEV)
        S.sparse_draft_attn(kv, qd, seq_d, ctx_t, sel, sel_stride, cnt, sl, nd, max_ctx, hq, w.sm_scale, out, lse, ws)
        return out, lse

    def do_unified(ws, vbx):
        sel, cnt, sl = _dev(sel_np, cnt_np, sl_np)
        out = torch.empty_like(q)
        lse = torch.empty(q.shape[0], hq, dtype=torch.float32, device=DEV)
        S.unified_attn(kv, q, ctx_t, bk, vbx, B, mv, max_ctx, hq, k, s, w.sm_scale, sel, sel_stride, cnt, sl,
                       out, lse, ws)
        return out, lse, sel, cnt, sl

    fresh = {}
    fv = do_verify(S.workspace(sizes["verify"]))
    fresh["verify"] = fv
    fresh["topk"] = do_topk(S.workspace(sizes["topk"]), fv[2], fv[1])
    fresh["draft"] = do_draft(S.workspace(sizes["draft"]))
    fresh["unified"] = do_unified(S.workspace(sizes["unified"]), vb)
    torch.cuda.synchronize()

    shared = S.workspace(max(sizes.values()))
    got = []
    v1 = do_verify(shared)
    got.append(("verify", v1, fresh["verify"]))
    got.append(("topk", do_topk(shared, v1[2], v1[1]), fresh["topk"]))
    got.append(("draft", do_draft(shared), fresh["draft"]))
    got.append(("unified", do_unified(shared, vb), fresh["unified"]))
    got.append(("verify again", do_verify(shared), fresh["verify"]))
    got.append(("unified again", do_unified(shared, vb), fresh["unified"]))
    torch.cuda.synchronize()
    assert S.read_device_error(shared) == 0
    def bits(t):   # compare bit patterns (NaN-safe, -0.0 != +0.0)
        return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)

    for name, a, b in got:
        for x, y in zip(a, b):
            assert torch.equal(bits(x), bits(y)), f"{name} differs from a fresh workspace"
    out_u, lse_u = got[3][1][0], got[3][1][1]
    o_ref, l_ref, _, _ = O.unified_step(bf16_tensor_to_f64(q), kp, vp, bt, ctx, isv, k, s, w.sm_scale, sels0, sl_np)
    assert_attn_close(bf16_tensor_to_f64(out_u), o_ref, "shared-ws unified O")
    assert_lse_close(lse_u.cpu().numpy(), l_ref, "shared-ws unified LSE")


def test_verify_over_512_requests_twice(S):
    """A verify call of 600 requests runs as a piece of 512 and one of 88 on
    one workspace layout; the same call made twice on one workspace gives the
    same bits, and sampled requests of both pieces match the oracle."""
    say("[ws pieces] verify n=600 twice")
    hq, hkv, k = 4, 2, 4
    rng = np.random.default_rng(5)
    lengths = rng.integers(40, 2600, size=600)
    w = make_workload(dict(hq=hq, hkv=hkv, k=k, s=0.05, batch=600), seed=62, lengths=lengths)
    kv = _kv(S, w)
    n = w.batch
    max_ctx = int(w.caps.max())
    lstride = -(-max_ctx // 16) * 16
    q = w.qbank[:, : k + 1].contiguous().to(DEV)
    seq = torch.arange(n, dtype=torch.int32, device=DEV)
    ctx = torch.as_tensor(lengths.astype(np.int32), device=DEV)
    ws = S.workspace(S.verify_workspace_size(n, max_ctx, hq, hkv, k))
    res = []
    for rep in range(2):
        out = torch.full_like(q, 7)
        lse = torch.full((n, k + 1, hq), 7.0, dtype=torch.float32, device=DEV)
        lg = torch.empty(n, hkv, lstride // 16, S.dump_pitch(hq, hkv, k), 16, dtype=torch.float32, device=DEV)
        S.verify_attn(kv, q, seq, ctx, n, max_ctx, hq, k, w.sm_scale, out, lse, lg, lstride, ws)
        torch.cuda.synchronize()
        assert S.read_device_error(ws) == 0
        res.append((out, lse))
    assert torch.equal(res[0][0].view(torch.int16), res[1][0].view(torch.int16))
    assert torch.equal(res[0][1], res[1][1])
    kp, vp, bt = host_pages(w)
    q64, o64, lse_h = bf16_tensor_to_f64(q), bf16_tensor_to_f64(res[1][0]), res[1][1].cpu().numpy()
    for r in [0, 1, 255, 511, 512, 513, 550, 599] + [int(x) for x in np.argsort(lengths)[-4:]]:
        kc, vc = request_kv(kp, vp, bt, r, int(lengths[r]))
        o_ref, l_ref, _ = O.verify_attention(q64[r], kc, vc, w.sm_scale)
        assert_attn_close(o64[r], o_ref, f"600-verify O r={r}")
        assert_lse_close(lse_h[r], l_ref, f"600-verify LSE r={r}")


# ---------------------------------------------------- non-finite pool row 0
def test_nonfinite_page0_never_reaches_outputs(S):
    """Masked draft positions (tile padding past a set's end, indices outside
    the context) load pool row 0 and must contribute exactly nothing: with
    physical page 0 unused by every request and filled with NaN and inf, a
    unified launch (verifies and drafts) matches the oracle."""
    say("[page0 poison] unified launch with NaN/inf in physical page 0")
    hq, hkv, k, s = 32, 8, 8, 0.05
    lengths = [700, 1500, 333, 2100, 1250, 950, 1800, 420, 2600, 1100]
    w = make_workload(dict(hq=hq, hkv=hkv, k=k, s=s, batch=len(lengths)), seed=71, lengths=lengths,
                      extra_pages=1)
    bt = w.block_table.clone()
    used = set()
    for r in range(w.batch):
        used.update(bt[r, : -(-int(w.caps[r]) // 16)].tolist())
    free = [p for p in range(w.num_pages) if p not in used]
    assert len(free) == 1
    if 0 in used:   # move page 0's owner to the free page
        r, j = [(int(a), int(b)) for a, b in zip(*np.nonzero(bt.numpy() == 0))
                if b < -(-int(w.caps[int(a)]) // 16)][0]
        w.k_pages[free[0]] = w.k_pages[0]
        w.v_pages[free[0]] = w.v_pages[0]
        bt[r, j] = free[0]
    w.block_table = bt
    poison = torch.tensor([float("nan"), float("inf"), -float("inf")], dtype=torch.bfloat16)
    w.k_pages[0] = poison.repeat(hkv * 16 * 128 // 3 + 1)[: hkv * 16 * 128].view(hkv, 16, 128).to(w.k_pages.device)
    w.v_pages[0] = poison.repeat(hkv * 16 * 128 // 3 + 1)[: hkv * 16 * 128].view(hkv, 16, 128).to(w.v_pages.device)
    kp, vp, btn = host_pages(w)
    sels0 = _oracle_sels(w, kp, vp, btn)
    B = w.batch
    max_ctx = int(w.caps.max())
    sel_stride = O.select_count(max_ctx, s)
    mv = int(np.bincount(w.bucket_ids).max())
    kv = _kv(S, w)
    ws = S.workspace(S.unified_workspace_size(B, mv, max_ctx, hq, hkv, k))
    for t in (1, 4):
        vb, isv, ctx, step = cycle_state(w, t)
        sel_np, cnt_np = _sel_arrays(sels0, B, hkv, sel_stride)
        sl_np = w.verify_lens.astype(np.int32)
        sel, cnt, sl = _dev(sel_np, cnt_np, sl_np)
        q = pack_rows(w, isv, step, DEV)
        out = torch.empty_like(q)
        lse = torch.empty(q.shape[0], hq, dtype=torch.float32, device=DEV)
        S.unified_attn(kv, q, torch.from_numpy(ctx.astype(np.int32)).to(DEV), torch.from_numpy(w.bucket_ids).to(DEV),
                       vb, B, mv, max_ctx, hq, k, s, w.sm_scale, sel, sel_stride, cnt, sl, out, lse, ws)
        torch.cuda.synchronize()
        assert S.read_device_error(ws) == 0
        o_ref, l_ref, _, _ = O.unified_step(bf16_tensor_to_f64(q), kp, vp, btn, ctx, isv, k, s, w.sm_scale,
                                            sels0, sl_np)
        assert_attn_close(bf16_tensor_to_f64(out), o_ref, f"page0-poison O t={t}")
        assert_lse_close(lse.cpu().numpy(), l_ref, f"page0-poison LSE t={t}")


# ------------------------------------------------------- device error bits
def test_verify_short_and_seq_range_flag_and_skip(S):
    """A verify context shorter than k+1 (SSPEC_DEV_ERR_VERIFY_SHORT) and a
    request id outside [0, num_seqs) (SSPEC_DEV_ERR_SEQ_RANGE): the item is
    skipped (its outputs untouched) and the other items stay exact."""
    say("[error bits] VERIFY_SHORT, SEQ_RANGE")
    hq, hkv, k = 16, 8, 8
    lengths = [700, 1500, 900]
    w = make_workload(dict(hq=hq, hkv=hkv, k=k, s=0.05, batch=3), seed=81, lengths=lengths)
    kv = _kv(S, w)
    n = 3
    max_ctx = int(w.caps.max())
    lstride = -(-max_ctx // 16) * 16
    q = w.qbank[:, : k + 1].contiguous().to(DEV)
    kp, vp, bt = host_pages(w)
    q64 = bf16_tensor_to_f64(q)
    ws = S.workspace(S.verify_workspace_size(n, max_ctx, hq, hkv, k))
    lg = torch.empty(n, hkv, lstride // 16, S.dump_pitch(hq, hkv, k), 16, dtype=torch.float32, device=DEV)
    for bit, seq_l, ctx_l, bad in (("VERIFY_SHORT", [0, 1, 2], [700, k, 900], 1),
                                   ("SEQ_RANGE", [0, 99, 2], lengths, 1),
                                   ("SEQ_RANGE", [0, 1, -1], lengths, 2)):
        out = torch.full_like(q, 7)
        lse = torch.full((n, k + 1, hq), 7.0, dtype=torch.float32, device=DEV)
        seq = torch.as_tensor(seq_l, dtype=torch.int32, device=DEV)
        ctx = torch.as_tensor(ctx_l, dtype=torch.int32, device=DEV)
        S.verify_attn(kv, q, seq, ctx, n, max_ctx, hq, k, w.sm_scale, out, lse, lg, lstride, ws)
        torch.cuda.synchronize()
        assert S.read_device_error(ws) == S.DEV_ERR[bit], bit
        assert bool((lse[bad] == 7.0).all()) and bool((out[bad].float() == 7.0).all()), f"{bit}: skipped item written"
        for r in range(n):
            if r == bad:
                continue
            kc, vc = request_kv(kp, vp, bt, r, lengths[r])
            o_ref, l_ref, _ = O.verify_attention(q64[r], kc, vc, w.sm_scale)
            assert_attn_close(bf16_tensor_to_f64(out)[r], o_ref, f"{bit} neighbour O r={r}")
            assert_lse_close(lse.cpu().numpy()[r], l_ref, f"{bit} neighbour LSE r={r}")


def test_draft_selection_errors_and_empty_set(S):
    """Draft requests whose selection holds a negative index, or a sel_count
    above sel_stride, raise SSPEC_DEV_ERR_SEL_RANGE; an index at or past
    sel_len (what a rollback leaves) is left out silently.  The results
    equal the oracle over the remaining set.  A request with no selected
    token and no tail attends to nothing: O = 0, LSE = -inf."""
    say("[error bits] SEL_RANGE, empty draft set")
    hq, hkv, s = 32, 8, 0.05
    lengths = [1500, 2100, 900, 1200]
    w = make_workload(dict(hq=hq, hkv=hkv, k=8, s=s, batch=4), seed=82, lengths=lengths)
    kp, vp, bt = host_pages(w)
    sels = _oracle_sels(w, kp, vp, bt)
    n = 4
    max_ctx = int(w.caps.max())
    sel_stride = O.select_count(max_ctx, s)
    sel_np, cnt_np = _sel_arrays(sels, n, hkv, sel_stride)
    sl_np = w.verify_lens.astype(np.int32)
    ctx_np = sl_np + np.array([2, 3, 1, 0], np.int32)
    sel_np[0, 0, 5] = int(sl_np[0]) + 5          # past sel_len
    sel_np[0, 3, 0] = -3                          # negative
    cnt_np[1] = sel_stride + 40                   # more than the row holds: clamped to sel_stride
    sel_np[1, :, O.select_count(int(sl_np[1]), s):] = int(sl_np[1]) + 100   # ... whose tail entries are out of range
    cnt_np[3] = 0                                 # empty set, no tail (ctx == sel_len)
    qd = torch.stack([w.qbank[r, 9] for r in range(n)]).contiguous().to(DEV)
    kv = _kv(S, w)
    out = torch.empty_like(qd)
    lse = torch.empty(n, hq, dtype=torch.float32, device=DEV)
    ws = S.workspace(S.draft_workspace_size(n, max_ctx, hq, hkv))
    sel, cnt, sl, ctx = _dev(sel_np, cnt_np, sl_np, ctx_np)
    S.sparse_draft_attn(kv, qd, torch.arange(n, dtype=torch.int32, device=DEV), ctx, sel, sel_stride, cnt, sl, n,
                        max_ctx, hq, w.sm_scale, out, lse, ws)
    torch.cuda.synchronize()
    assert S.read_device_error(ws) == S.DEV_ERR["SEL_RANGE"]
    o64, lse_h, q64 = bf16_tensor_to_f64(out), lse.cpu().numpy(), bf16_tensor_to_f64(qd)
    for r in range(3):
        c = int(ctx_np[r])
        kc, vc = request_kv(kp, vp, bt, r, c)
        m = min(int(cnt_np[r]), sel_stride)
        sets = [sel_np[r, h, :m][sel_np[r, h, :m] >= 0] for h in range(hkv)]
        o_ref, l_ref = O.sparse_draft_attention(q64[r], kc, vc, sets, int(sl_np[r]), c, w.sm_scale)
        assert_attn_close(o64[r], o_ref, f"sel-range draft O r={r}")
        assert_lse_close(lse_h[r], l_ref, f"sel-range draft LSE r={r}")
    assert np.all(o64[3] == 0.0), "empty draft set: O must be 0"
    assert np.all(np.isneginf(lse_h[3])), "empty draft set: LSE must be -inf"


def test_unified_without_verifying_requests(S):
    """A unified launch whose verify bucket holds no request: every request
    drafts, nothing is selected, results match the oracle."""
    say("[unified] no verifying request")
    hq, hkv, k, s = 32, 8, 8, 0.05
    lengths = [1200, 2600, 333, 4100, 1800, 950, 2222]
    w = make_workload(dict(hq=hq, hkv=hkv, k=k, s=s, batch=len(lengths)), seed=83, lengths=lengths)
    kp, vp, bt = host_pages(w)
    sels0 = _oracle_sels(w, kp, vp, bt)
    B = w.batch
    max_ctx = int(w.caps.max())
    sel_stride = O.select_count(max_ctx, s)
    _, isv, ctx, step = cycle_state(w, 3)
    step = np.where(isv, 1, step)
    ctx = w.verify_lens + step
    isv = np.zeros(B, bool)
    sel_np, cnt_np = _sel_arrays(sels0, B, hkv, sel_stride)
    sl_np = w.verify_lens.astype(np.int32)
    sel, cnt, sl = _dev(sel_np, cnt_np, sl_np)
    q = pack_rows(w, isv, step, DEV)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[0], hq, dtype=torch.float32, device=DEV)
    kv = _kv(S, w)
    ws = S.workspace(S.unified_workspace_size(B, 2, max_ctx, hq, hkv, k))
    S.unified_attn(kv, q, torch.from_numpy(ctx.astype(np.int32)).to(DEV), torch.from_numpy(w.bucket_ids).to(DEV),
                   k + 1, B, 2, max_ctx, hq, k, s, w.sm_scale, sel, sel_stride, cnt, sl, out, lse, ws)
    torch.cuda.synchronize()
    assert S.read_device_error(ws) == 0
    o_ref, l_ref, _, _ = O.unified_step(bf16_tensor_to_f64(q), kp, vp, bt, ctx, isv, k, s, w.sm_scale, sels0, sl_np)
    assert_attn_close(bf16_tensor_to_f64(out), o_ref, "no-verify unified O")
    assert_lse_close(lse.cpu().numpy(), l_ref, "no-verify unified LSE")
    assert np.array_equal(sel.cpu().numpy(), sel_np) and np.array_equal(sl.cpu().numpy(), sl_np)


# --------------------------------------------------------- partial residency
def test_unified_beside_gemms_on_another_stream(S):
    """torch GEMMs queued on a second stream (default priority) hold CUs when
    each unified launch starts, so its work-groups become resident at
    different times; every launch must still give the bits of a launch on
    an idle GPU, with no device error."""
    say("[unified] concurrent GEMMs on a second stream")
    hq, hkv, k, s = 32, 8, 8, 0.05
    lengths = [1300, 2500, 900, 3300, 1700, 2100, 600, 1900, 2800, 1100, 5000, 7000, 3900, 4400]
    w = make_workload(dict(hq=hq, hkv=hkv, k=k, s=s, batch=len(lengths)), seed=84, lengths=lengths)
    kv = _kv(S, w)
    B = w.batch
    max_ctx = int(w.caps.max())
    sel_stride = O.select_count(max_ctx, s)
    mv = int(np.bincount(w.bucket_ids).max())
    rng = np.random.default_rng(2)
    sel_np = np.zeros((B, hkv, sel_stride), np.int32)
    cnt_np = np.zeros(B, np.int32)
    for r in range(B):
        L = int(w.verify_lens[r])
        K = O.select_count(L, s)
        cnt_np[r] = K
        for h in range(hkv):
            sel_np[r, h, :K] = np.sort(rng.choice(L, K, replace=False))
    sl_np = w.verify_lens.astype(np.int32)
    vb, isv, ctx, step = cycle_state(w, 0)
    q = pack_rows(w, isv, step, DEV)
    ctx_t = torch.from_numpy(ctx.astype(np.int32)).to(DEV)
    bk = torch.from_numpy(w.bucket_ids).to(DEV)
    ws = S.workspace(S.unified_workspace_size(B, mv, max_ctx, hq, hkv, k))

    def launch():
        sel, cnt, sl = _dev(sel_np, cnt_np, sl_np)
        out = torch.empty_like(q)
        lse = torch.empty(q.shape[0], hq, dtype=torch.float32, device=DEV)
        S.unified_attn(kv, q, ctx_t, bk, vb, B, mv, max_ctx, hq, k, s, w.sm_scale, sel, sel_stride, cnt, sl,
                       out, lse, ws)
        return out, lse, sel

    ref = launch()
    torch.cuda.synchronize()
    assert S.read_device_error(ws) == 0
    a = torch.randn(4096, 4096, dtype=torch.bfloat16, device=DEV)
    b = torch.randn(4096, 4096, dtype=torch.bfloat16, device=DEV)
    side = torch.cuda.Stream()
    for rep in range(6):
        torch.cuda.synchronize()
        with torch.cuda.stream(side):
            for _ in range(4):
                c = a @ b
        got = launch()
        torch.cuda.synchronize()
        assert S.read_device_error(ws) == 0, f"rep {rep}"
        assert torch.equal(got[0].view(torch.int16), ref[0].view(torch.int16)), f"rep {rep}: O differs"
        assert torch.equal(got[1], ref[1]) and torch.equal(got[2], ref[2]), f"rep {rep}"
    del c


# ------------------------------------------------------------ Top-K paths
def _topk_from_rows(S, lg_rows, lse_ref, hq, hkv, k, L, s):
    lstride = -(-L // 16) * 16
    lg = rows_to_dump(lg_rows.astype(np.float32), hkv, k, lstride, S.dump_pitch(hq, hkv, k))[None]
    logits = torch.from_numpy(lg).to(DEV)
    lse = torch.from_numpy(lse_ref[None].astype(np.float32)).to(DEV)
    K = O.select_count(L, s)
    sel = torch.full((1, hkv, K), -1, dtype=torch.int32, device=DEV)
    cnt = torch.zeros(1, dtype=torch.int32, device=DEV)
    sl = torch.zeros(1, dtype=torch.int32, device=DEV)
    ws = S.workspace(S.pillar_topk_workspace_size(1, L, hkv))
    before = selection_paths(ws)
    S.pillar_topk(logits, lse, lstride, torch.zeros(1, dtype=torch.int32, device=DEV),
                  torch.tensor([L], dtype=torch.int32, device=DEV), 1, 1, L, hq, hkv, k, s, sel, K, cnt, sl, ws)
    torch.cuda.synchronize()
    assert S.read_device_error(ws) == 0
    return sel.cpu().numpy()[0], int(cnt.cpu()[0]), selection_paths(ws) - before


@pytest.mark.parametrize("case", ["bitmap", "bitmap-long", "bin-collect", "global-passes"])
def test_topk_paths(S, case):
    """Score rows built so that each Top-K path must run (which one is
    derived on the host from the scores' float32 bit patterns, and read back
    from the workspace's per-path counts): the pillar workload's rows at 3001
    and at 9001 keys (bitmaps, over two and five score chunks), a
    row whose K-th key sits in a bin of 3000 keys (more than 2048: collection
    of the bin), and a flat row of 10000 equal scores (the
    threshold bin holds every key: two global passes, ties to the lowest
    indices)."""
    say(f"[topk path] {case}")
    rng = np.random.default_rng(9)
    if case.startswith("bitmap"):
        hq, hkv, k, s = 16, 4, 5, 0.05
        L = 3001 if case == "bitmap" else 9001
        q = rng.standard_normal((k + 1, hq, 128))
        kc = rng.standard_normal((hkv, L, 128))
        vc = rng.standard_normal((hkv, L, 128))
        _, lse_ref, lg_ref = O.verify_attention(q, kc, vc, 1 / math.sqrt(128))
        want = 0
    else:
        hq, hkv, k = 2, 2, 0
        if case == "bin-collect":
            # softmax weights: 3000 keys decreasing inside [1.02, 1.10) * 2^-12
            # (one 11-bit bin, 2% from its edges), the other 9000 equal and
            # far smaller; K = 1200 falls in that bin
            L, s = 12000, 0.1
            w8 = np.empty(L)
            w8[:3000] = 2.0 ** -12 * (1.10 - 0.08 * np.arange(3000) / 3000)
            w8[3000:] = (1.0 - w8[:3000].sum()) / (L - 3000)
            row = np.log(w8)
        else:
            L, s = 10000, 0.05
            row = np.zeros(L)
        lg_ref = np.broadcast_to(row, (hq, 1, L)).astype(np.float64).copy()
        m = row.max()
        lse_ref = np.full((1, hq), m + math.log(np.exp(row - m).sum()))
        want = 1 if case == "bin-collect" else 2
    S_ref = O.pillar_scores(lg_ref, lse_ref, hkv)
    sel_ref, K = O.pillar_topk(lg_ref, lse_ref, hkv, s)
    for h in range(hkv):
        assert expected_path(S_ref[h].astype(np.float32), K) == want, "case does not reach its path"
    sel, cnt, paths = _topk_from_rows(S, lg_ref, lse_ref, hq, hkv, k, L, s)
    assert paths[want] == hkv and paths.sum() == hkv, f"paths taken {paths.tolist()}"
    for h in range(hkv):
        check_topk(sel[h], cnt, S_ref[h], sel_ref[h], f"{case} h={h}")
    if not case.startswith("bitmap"):
        assert np.array_equal(sel[0], np.arange(K)), "expected the K first (highest / lowest-index) keys"

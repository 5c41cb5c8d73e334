"""The naive-batching baseline (sspec_unified_attn_naive) against the oracle
and against the fused launch.

Naive batching runs every item of the unified batch in the verify's tile
shape: a draft fills G of the G*(k+1) query columns and is cut into the
launch's verify chunk length.  Its verifies and selections must equal the
fused launch's bit for bit (same tasks, same arithmetic); its drafts must
match the oracle like every other draft.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle as O
from sspec_workload import cycle_state, make_workload, pack_rows
from tests.helpers import assert_attn_close, assert_lse_close, bf16_tensor_to_f64, host_pages, say
from tests.test_parity_gpu import _kv, _oracle_selection_state

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def S():
    from sparse_self_speculative_amd import sspec
    return sspec


NAIVE_CASES = [
    # (hq, hkv, k, s, lengths)
    (32, 8, 8, 0.05, [1200, 2600, 333, 4100, 1800, 950, 2222, 1500, 3000, 64, 2048, 1700]),  # 3 query tiles
    (16, 8, 8, 0.1, [500, 1030, 2047, 33, 800, 1600, 700, 2900]),                            # 2 tiles
    (48, 8, 7, 0.05, [1500, 2900, 1000, 2000, 2500, 1200, 600, 3100]),                       # G*(k+1) = 48
    (8, 8, 8, 0.05, [900, 1700, 2500, 400, 1300]),                                           # G = 1: 1 tile
    (32, 8, 8, 1.0, [1200, 2600, 333, 1800, 950, 2222, 1500, 640, 3000, 1100]),              # drafts > 1 chunk
]


def _launch(S, fn, w, kv, ws, isv, step, ctx, vb, sels0, max_verify, max_ctx, sel_stride):
    B, hq, hkv, k, s = w.batch, w.num_q_heads, w.num_kv_heads, w.k, w.s
    sel_np = np.zeros((B, hkv, sel_stride), np.int32)
    for r in range(B):
        sel_np[r, :, : sels0[r].shape[1]] = sels0[r]
    cnt_np = np.array([sels0[r].shape[1] for r in range(B)], np.int32)
    sl_np = w.verify_lens.astype(np.int32)
    sel_t, cnt_t, sl_t = (torch.from_numpy(a).to(DEV) for a in (sel_np, cnt_np, sl_np))
    q = pack_rows(w, isv, step, DEV)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[0], hq, dtype=torch.float32, device=DEV)
    fn(kv, q, torch.from_numpy(ctx.astype(np.int32)).to(DEV), torch.from_numpy(w.bucket_ids).to(DEV), vb, B,
       max_verify, max_ctx, hq, k, s, w.sm_scale, sel_t, sel_stride, cnt_t, sl_t, out, lse, ws)
    torch.cuda.synchronize()
    assert S.read_device_error(ws) == 0
    return q, out, lse, sel_t.cpu().numpy(), cnt_t.cpu().numpy(), sl_t.cpu().numpy(), sl_np


@pytest.mark.parametrize("hq,hkv,k,s,lengths", NAIVE_CASES)
def test_naive_batching_parity(S, hq, hkv, k, s, lengths):
    say(f"[naive] hq={hq} hkv={hkv} k={k} s={s} B={len(lengths)}")
    w = make_workload(dict(hq=hq, hkv=hkv, k=k, s=s, batch=len(lengths)), seed=11 + hq + k, lengths=lengths)
    kp, vp, bt = host_pages(w)
    B = w.batch
    sels0 = _oracle_selection_state(w, kp, vp, bt)
    max_ctx = int(w.caps.max())
    sel_stride = O.select_count(max_ctx, s)
    max_verify = int(np.bincount(w.bucket_ids).max())
    kv = _kv(S, w)
    size = S.unified_workspace_size(B, max_verify, max_ctx, hq, hkv, k)
    ws_f, ws_n = S.workspace(size), S.workspace(size)
    for t in [0, k]:
        vb, isv, ctx, step = cycle_state(w, t)
        say(f"   launch t={t} verify_bucket={vb} n_verify={int(isv.sum())}")
        args = (w, kv, None, isv, step, ctx, vb, sels0, max_verify, max_ctx, sel_stride)
        q, out_f, lse_f, sel_f, cnt_f, sl_f, _ = _launch(S, S.unified_attn, *args[:2], ws_f, *args[3:])
        _, out_n, lse_n, sel_n, cnt_n, sl_n, sl0 = _launch(S, S.unified_attn_naive, *args[:2], ws_n, *args[3:])
        # verifies and selections: the same tasks as the fused launch, bit for bit
        nr = np.where(isv, k + 1, 1)
        off = np.concatenate([[0], np.cumsum(nr)])
        vrows = np.concatenate([np.arange(off[r], off[r + 1]) for r in np.nonzero(isv)[0]] or [np.zeros(0, int)])
        vrows_t = torch.from_numpy(vrows.astype(np.int64)).to(DEV)
        assert torch.equal(out_n[vrows_t], out_f[vrows_t]), "verify O differs from the fused launch"
        assert torch.equal(lse_n[vrows_t], lse_f[vrows_t]), "verify LSE differs from the fused launch"
        assert np.array_equal(sel_n, sel_f) and np.array_equal(cnt_n, cnt_f) and np.array_equal(sl_n, sl_f)
        # every row against the oracle
        o_ref, l_ref, _, sl_ref = O.unified_step(bf16_tensor_to_f64(q), kp, vp, bt, ctx, isv, k, s, w.sm_scale,
                                                 sels0, sl0)
        assert_attn_close(bf16_tensor_to_f64(out_n), o_ref, f"naive O t={t}")
        assert_lse_close(lse_n.cpu().numpy(), l_ref, f"naive LSE t={t}")
        assert np.array_equal(sl_n, sl_ref)


def test_naive_rejects_wide_tiles(S):
    """G*(k+1) = 68 (five query tiles) has no naive form: rejected on the host."""
    say("[naive] G*(k+1) = 68 rejected")
    w = make_workload(dict(hq=32, hkv=8, k=16, s=0.05, batch=2), seed=3, lengths=[600, 700])
    kv = _kv(S, w)
    ws = S.workspace(S.unified_workspace_size(2, 2, 800, 32, 8, 16))
    q = torch.zeros(2 * 17, 32, 128, dtype=torch.bfloat16, device=DEV)
    i32 = lambda *shape: torch.zeros(*shape, dtype=torch.int32, device=DEV)
    with pytest.raises(RuntimeError, match="naive"):
        S.unified_attn_naive(kv, q, i32(2), i32(2), 0, 2, 2, 800, 32, 16, 0.05, w.sm_scale, i32(2, 8, 40), 40,
                             i32(2), i32(2), torch.empty_like(q), torch.empty(34, 32, device=DEV), ws)

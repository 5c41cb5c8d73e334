"""The allocation-free entry point sspec_pillar_topk_noalloc (the library's
static scratch as workspace) against sspec_pillar_topk with a workspace of
its own: the same selections bit for bit, on two calls in a row, the second
with fewer and shorter requests (the scratch keeps the first call's
contents), and a clear rejection of a call too large for the scratch.
"""

from __future__ import annotations

import ctypes
import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from tests import abi_validation as V  # noqa: E402

LIB = os.path.join(ROOT, "sparse_self_speculative_amd", "libsspec.so")


def test_noalloc_rejects_calls_beyond_its_scratch():
    """No GPU needed: the size check precedes any HIP call."""
    lib = V.bind(LIB)
    f = lib.sspec_pillar_topk_noalloc
    f.argtypes = [V.P, V.P, V.I64, V.P, V.P, V.I32, V.I32, V.I32, V.I32, V.I32, V.I32, V.F64, V.P, V.I32,
                  V.P, V.P, V.P]
    need = lib.sspec_pillar_topk_workspace_size(512, 1 << 20, 8)
    assert need > (64 << 20)
    a = V.ADDR
    rc = f(a["logits"], a["lse"], 1 << 20, a["seq"], a["ctx"], 512, 512, 1 << 20, 32, 8, 8, 0.05, a["sel"],
           52429, a["cnt"], a["sl"], None)
    msg = lib.sspec_last_error().decode()
    assert rc == V.WORKSPACE and "static scratch" in msg and str(need) in msg, (rc, msg)
    # argument errors are still reported as such
    rc = f(a["logits"], a["lse"], 1 << 20, a["seq"], a["ctx"], 4, 512, 1 << 20, 32, 8, 8, 1.5, a["sel"],
           52429, a["cnt"], a["sl"], None)
    assert rc == V.INVALID


@pytest.mark.gpu
def test_noalloc_matches_workspace_entry_point():
    import torch

    import oracle as O
    from sparse_self_speculative_amd import sspec as S
    from sspec_workload import make_workload
    from tests.helpers import bf16_tensor_to_f64, check_topk, host_pages, request_kv, say

    dev = "cuda"
    for call, (hq, hkv, k, s, lengths) in enumerate([(32, 8, 8, 0.05, [5200, 1500, 3001, 77]),
                                                     (16, 8, 4, 0.1, [900, 1400])]):
        say(f"[noalloc] call {call}: hq={hq} hkv={hkv} k={k} s={s} L={lengths}")
        w = make_workload(dict(hq=hq, hkv=hkv, k=k, s=s, batch=len(lengths)), seed=90 + call, lengths=lengths)
        n = w.batch
        max_ctx = int(w.caps.max())
        lstride = -(-max_ctx // 16) * 16
        kv = S.PagedKV(w.k_pages.to(dev), w.v_pages.to(dev), w.block_table.to(dev))
        q = w.qbank[:, : k + 1].contiguous().to(dev)
        seq = torch.arange(n, dtype=torch.int32, device=dev)
        ctx = torch.as_tensor(np.asarray(lengths, np.int32), device=dev)
        out = torch.empty_like(q)
        lse = torch.empty(n, k + 1, hq, dtype=torch.float32, device=dev)
        lg = torch.empty(n, hkv, lstride // 16, S.dump_pitch(hq, hkv, k), 16, dtype=torch.float32, device=dev)
        wsv = S.workspace(S.verify_workspace_size(n, max_ctx, hq, hkv, k))
        S.verify_attn(kv, q, seq, ctx, n, max_ctx, hq, k, w.sm_scale, out, lse, lg, lstride, wsv)
        sel_stride = O.select_count(max_ctx, s)
        res = []
        for noalloc in (False, True):
            sel = torch.full((n, hkv, sel_stride), -5, dtype=torch.int32, device=dev)
            cnt = torch.zeros(n, dtype=torch.int32, device=dev)
            sl = torch.zeros(n, dtype=torch.int32, device=dev)
            if noalloc:
                S.pillar_topk_noalloc(lg, lse, lstride, seq, ctx, n, n, max_ctx, hq, hkv, k, s, sel, sel_stride,
                                      cnt, sl)
            else:
                ws = S.workspace(S.pillar_topk_workspace_size(n, max_ctx, hkv))
                S.pillar_topk(lg, lse, lstride, seq, ctx, n, n, max_ctx, hq, hkv, k, s, sel, sel_stride, cnt, sl,
                              ws)
            torch.cuda.synchronize()
            res.append((sel.cpu(), cnt.cpu(), sl.cpu()))
        assert S.read_device_error(wsv) == 0
        for a, b in zip(*res):
            assert torch.equal(a, b), f"call {call}: noalloc differs from the workspace entry point"
        # and both against the oracle
        kp, vp, bt = host_pages(w)
        q64 = bf16_tensor_to_f64(q)
        sel_h, cnt_h = res[1][0].numpy(), res[1][1].numpy()
        for r, L in enumerate(lengths):
            kc, vc = request_kv(kp, vp, bt, r, L)
            _, lse_ref, lg_ref = O.verify_attention(q64[r], kc, vc, w.sm_scale)
            S_ref = O.pillar_scores(lg_ref, lse_ref, hkv)
            sel_ref, K = O.pillar_topk(lg_ref, lse_ref, hkv, s)
            for h in range(hkv):
                check_topk(sel_h[r, h], int(cnt_h[r]), S_ref[h], sel_ref[h], f"noalloc call {call} r={r} h={h}")

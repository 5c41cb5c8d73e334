"""Shared helpers of the parity tests: run the oracle on host copies of the
seeded inputs and compare with the HIP path under the acceptance rules.

Acceptance (from the method's statement of the target):
  attention outputs  max |err| <= 1e-2 and mean |err| <= 1e-3 vs the oracle
  LSE                |err| <= 1e-3
  Top-K sets         equal except indices whose oracle score lies within
                     1e-4 (relative) of the oracle's K-th score; the GPU set
                     must hold exactly K unique ascending indices
  logit dump         |err| <= 1e-3 (internal check)
"""

from __future__ import annotations

import math
import sys

import numpy as np
import torch

import oracle as O
from sspec_workload import to_numpy_bf16

OUT_MAX, OUT_MEAN, LSE_TOL, DUMP_TOL, TIE_REL = 1e-2, 1e-3, 1e-3, 1e-3, 1e-4


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bf16_tensor_to_f64(t: torch.Tensor) -> np.ndarray:
    return O.bf16_to_f64(to_numpy_bf16(t))


def host_pages(w):
    return to_numpy_bf16(w.k_pages), to_numpy_bf16(w.v_pages), w.block_table.cpu().numpy()


def request_kv(kp, vp, bt, r, n_tokens, page=16):
    return O.gather_kv(kp, bt[r], n_tokens, page), O.gather_kv(vp, bt[r], n_tokens, page)


def assert_attn_close(got: np.ndarray, ref: np.ndarray, what: str):
    err = np.abs(got - ref)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    mx, mean = float(err.max()), float(err.mean())
    assert mx <= OUT_MAX and mean <= OUT_MEAN, f"{what}: max {mx:.3e} mean {mean:.3e}"
    return mx, mean


def assert_lse_close(got, ref, what):
    err = np.abs(np.asarray(got, np.float64) - ref)
    mx = float(err.max()) if err.size else 0.0
    assert mx <= LSE_TOL, f"{what}: LSE max err {mx:.3e}"
    return mx


def check_topk(sel_gpu: np.ndarray, K_gpu: int, S_ref: np.ndarray, sel_ref: np.ndarray, what: str):
    """Near-tie rule: the two sets may differ only in indices whose oracle
    score is within TIE_REL of the oracle's K-th score."""
    K = len(sel_ref)
    assert K_gpu == K, f"{what}: K {K_gpu} != {K}"
    g = np.asarray(sel_gpu[:K], dtype=np.int64)
    assert np.all(np.diff(g) > 0), f"{what}: GPU selection not strictly ascending"
    assert g.min() >= 0 and g.max() < S_ref.shape[0], f"{what}: index out of range"
    diff = np.setxor1d(g, sel_ref)
    if diff.size == 0:
        return 0
    sK = np.sort(S_ref)[::-1][K - 1]
    rel = np.abs(S_ref[diff] - sK) / max(sK, 1e-300)
    assert np.all(rel <= TIE_REL), \
        f"{what}: {diff.size} differing indices, worst rel gap {rel.max():.3e} (allowed {TIE_REL})"
    return int(diff.size)


def dump_to_rows(lg, hq, hkv, k, L):
    """Page-blocked dump of one item, float [hkv][stride/16][Mp][16] (or flat)
    -> rows [hq][k+1][L]."""
    G = hq // hkv
    lg = lg.reshape(hkv, -1, lg.shape[-1] if lg.ndim == 4 else 1, 16) if lg.ndim != 4 else lg
    nb = -(-L // 16)
    out = np.empty((hq, k + 1, L), lg.dtype)
    for g in range(hq):
        h, gi = divmod(g, G)
        rows = lg[h, :nb, gi * (k + 1): (gi + 1) * (k + 1), :]          # [blocks][k+1][16]
        out[g] = rows.transpose(1, 0, 2).reshape(k + 1, nb * 16)[:, :L]
    return out


def rows_to_dump(rows, hkv, k, stride, mp):
    """Rows [hq][k+1][L] -> page-blocked dump [hkv][stride/16][mp][16] (-inf elsewhere)."""
    hq, _, L = rows.shape
    G = hq // hkv
    lg = np.full((hkv, stride // 16, mp, 16), -np.inf, np.float32)
    nb = -(-L // 16)
    for g in range(hq):
        h, gi = divmod(g, G)
        pad = np.full((k + 1, nb * 16), -np.inf, np.float32)
        pad[:, :L] = rows[g]
        lg[h, :nb, gi * (k + 1): (gi + 1) * (k + 1), :] = pad.reshape(k + 1, nb, 16).transpose(1, 0, 2)
    return lg


def request_kv_dev(w, r, n_tokens):
    """float64 K, V [Hkv][n][d] of request r's first n tokens, copying only that
    request's pages to the host (for workloads too large to copy whole)."""
    pages = w.block_table[r, : -(-n_tokens // 16)].to(w.k_pages.device).long()
    kp = to_numpy_bf16(w.k_pages[pages])
    vp = to_numpy_bf16(w.v_pages[pages])
    row = np.arange(pages.shape[0])
    return O.gather_kv(kp, row, n_tokens, 16), O.gather_kv(vp, row, n_tokens, 16)


SEL_PATH_OFFSET = 32   # bytes: the workspace header's per-path selection counts (4 x uint32)


def selection_paths(ws: torch.Tensor) -> np.ndarray:
    """Selections run so far on a workspace, by Top-K path: [bitmaps,
    threshold-bin collection, two global passes, (unused)] (diagnostic
    header counts)."""
    torch.cuda.synchronize()
    return ws[SEL_PATH_OFFSET: SEL_PATH_OFFSET + 16].cpu().view(torch.int32).numpy().astype(np.int64)


def expected_path(S_ref_f32: np.ndarray, K: int) -> int:
    """Which Top-K path the kernel's branch conditions pick for a score row,
    derived from the scores' float32 bit patterns: 0 bitmaps (the 11-bit bin
    of the K-th largest key holds <= 2048 keys), 1 collection of that bin
    (<= 4096 keys), 2 two global passes."""
    bins = np.asarray(S_ref_f32, np.float32).view(np.uint32) >> 20
    hist = np.bincount(bins, minlength=2048)
    above = 0
    for b in range(2047, -1, -1):
        if above + hist[b] >= K:
            n1 = int(hist[b])
            break
        above += int(hist[b])
    if n1 <= 2048:
        return 0
    return 1 if n1 <= 4096 else 2

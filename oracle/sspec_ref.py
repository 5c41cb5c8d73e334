"""Plain CPU oracle of the SparseSpec attention hot path (float64 numpy).

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  The product path (the
HIP library and its Python binding) never calls it, and this module shares
no code, tables or constants with that path.

Source: the talk-notes page "Accelerating Large-Scale Reasoning Model
Inference with Sparse Self-Speculative Decoding" (MLSys 2026).  Citations
below name that page's sections (in English) and the paper anchors the
notes give, e.g. [PillarAttn, paper §4.1].

What is computed, and how it is pinned (tests/test_oracle_pins.py):
  * verify attention with a logit + LSE dump   -- pinned against torch's
    scaled_dot_product_attention / logsumexp, a closed form (all-zero keys)
    and the normalisation invariant.
  * score recovery and GQA/query averaging      -- pinned by closed forms
    (all-zero keys; one-hot attention per query head).
  * Top-K selection, lowest index on ties       -- pinned by exhaustive
    subset search on tiny inputs, the flat-score closed form and planted
    separable pillars.
  * sparse draft attention over the selection    -- pinned by s = 1.0 being
    full attention (torch SDPA) and by the uniform-attention closed form.
  * KV append through the block table, and the rollback of a verify's
    rejected tokens                              -- pinned by a contiguous
    block table read back with plain reshapes, paging invariance, the
    untouched rest of the pool, and the rollback's closed forms.
All functions are pinned; none is "parity unpinned".

Readings of points the pages leave open (each is listed in the design
notes): causal masking among the k+1 verify queries; the natural log for
LSE; logits scaled by sm_scale; the average taken over all k+1 verify
queries; K = min(L, ceil(s*L)) in IEEE double; the draft attends to the
selected tokens plus the tokens appended since the selection.

Arithmetic is float64 throughout; bfloat16 inputs are widened exactly.
"""

from __future__ import annotations

import math
from typing import List, Sequence, Tuple

import numpy as np


# ---------------------------------------------------------------- inputs ---

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64, exactly."""
    b = np.ascontiguousarray(bits).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def gather_kv(pages: np.ndarray, bt_row: np.ndarray, n_tokens: int,
              page_size: int) -> np.ndarray:
    """Read logical tokens [0, n_tokens) of one request out of a paged pool.

    pages: uint16 [num_pages][Hkv][page_size][d]; token j lives in physical
    page bt_row[j // page_size] at slot j % page_size.
    Returns float64 [Hkv][n_tokens][d].
    """
    j = np.arange(n_tokens)
    phys = np.asarray(bt_row)[j // page_size]
    rows = pages[phys, :, j % page_size, :]          # [n][Hkv][d]
    return bf16_to_f64(rows).transpose(1, 0, 2)


def select_count(L: int, s: float) -> int:
    """Number of critical tokens kept per KV head: K = min(L, ceil(s*L)),
    with s*L evaluated in IEEE double [PillarAttn, paper §4.1; s from
    Experimental setup, paper §5.4]."""
    return int(min(L, math.ceil(float(s) * float(L))))


# --------------------------------------------------------------- verify ---

def verify_attention(q: np.ndarray, kc: np.ndarray, vc: np.ndarray,
                     sm_scale: float) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Full attention of the k+1 verify queries of one request, with the
    logit and log-sum-exp dump [PillarAttn, paper §4.1: the verify kernel
    emits the attention scores as logits and LSE while it runs].

    q : float64 [k+1][Hq][d]   queries at positions L-k-1+i, i = 0..k
    kc, vc : float64 [Hkv][L][d]  the request's keys / values, L = ctx_len
    Query head g reads KV head g // (Hq/Hkv).  Query i sees keys j <= L-k-1+i.
    Returns O [k+1][Hq][d], lse [k+1][Hq] (natural log),
    logits [Hq][k+1][L] (sm_scale * q.k, -inf where masked).
    """
    kp1, hq, d = q.shape
    hkv, L, _ = kc.shape
    G = hq // hkv
    scale = float(np.float32(sm_scale))
    logits = np.full((hq, kp1, L), -np.inf)
    out = np.zeros((kp1, hq, d))
    lse = np.zeros((kp1, hq))
    for g in range(hq):
        h = g // G
        raw = q[:, g, :] @ kc[h].T                    # [k+1][L]
        for i in range(kp1):
            n_vis = L - kp1 + i + 1                   # keys 0 .. L-k-1+i
            row = scale * raw[i, :n_vis]
            logits[g, i, :n_vis] = row
            m = row.max()
            lse_i = m + math.log(np.exp(row - m).sum())
            p = np.exp(row - lse_i)
            out[i, g] = p @ vc[h, :n_vis]
            lse[i, g] = lse_i
    return out, lse, logits


# ------------------------------------------------------------ selection ---

def pillar_scores(logits: np.ndarray, lse: np.ndarray, num_kv_heads: int) -> np.ndarray:
    """Recovered attention scores averaged per KV head [PillarAttn, §4.1]:
    S[h, j] = mean over the query heads g of group h and the k+1 verify
    queries i of exp(logits[g, i, j] - lse[i, g]); masked entries give 0.

    logits [Hq][k+1][L], lse [k+1][Hq] -> S float64 [Hkv][L].
    """
    hq, kp1, L = logits.shape
    G = hq // num_kv_heads
    probs = np.exp(logits - lse.T[:, :, None])        # exp(-inf) = 0
    S = np.zeros((num_kv_heads, L))
    for h in range(num_kv_heads):
        S[h] = probs[h * G:(h + 1) * G].reshape(G * kp1, L).mean(axis=0)
    return S


def topk_lowest_index(scores: np.ndarray, K: int) -> np.ndarray:
    """Indices of the K largest scores, exact ties going to the lower index,
    returned in ascending index order."""
    L = scores.shape[0]
    order = np.lexsort((np.arange(L), -scores))     # score desc, then index asc
    return np.sort(order[:K]).astype(np.int64)


def pillar_topk(logits: np.ndarray, lse: np.ndarray, num_kv_heads: int,
                s: float) -> Tuple[np.ndarray, int]:
    """Critical-token selection of one verify request [PillarAttn, §4.1]:
    average the recovered scores, keep K = ceil(s*L) tokens per KV head.
    Returns (sel int64 [Hkv][K] ascending, K)."""
    L = logits.shape[2]
    K = select_count(L, s)
    S = pillar_scores(logits, lse, num_kv_heads)
    sel = np.stack([topk_lowest_index(S[h], K) for h in range(num_kv_heads)])
    return sel, K


# ---------------------------------------------------------------- draft ---

def draft_token_set(sel_h: np.ndarray, sel_len: int, ctx_len: int) -> np.ndarray:
    """Tokens one draft query attends to for one KV head: the selected
    critical tokens that are still in the context, plus every token appended
    since the selection was taken (positions [sel_len, ctx_len))
    [PillarAttn, §4.1: only the critical tokens are loaded; the pattern is
    refreshed every k steps, paper Fig. 7]."""
    lim = min(sel_len, ctx_len)
    kept = np.asarray(sel_h)[np.asarray(sel_h) < lim]
    tail = np.arange(sel_len, ctx_len) if ctx_len > sel_len else np.zeros(0, np.int64)
    return np.union1d(kept, tail).astype(np.int64)


def sparse_draft_attention(q: np.ndarray, kc: np.ndarray, vc: np.ndarray,
                           sel: Sequence[np.ndarray], sel_len: int, ctx_len: int,
                           sm_scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """One draft query (position ctx_len-1) attending to its KV head's token
    set only [PillarAttn, §4.1].

    q : float64 [Hq][d]; kc, vc : float64 [Hkv][>=ctx_len][d];
    sel[h] : selected indices of KV head h.
    Returns O [Hq][d], lse [Hq].
    """
    hq, d = q.shape
    hkv = kc.shape[0]
    G = hq // hkv
    scale = float(np.float32(sm_scale))
    out = np.zeros((hq, d))
    lse = np.zeros(hq)
    for h in range(hkv):
        A = draft_token_set(sel[h], sel_len, ctx_len)
        for g in range(h * G, (h + 1) * G):
            row = scale * (kc[h, A] @ q[g])
            m = row.max()
            lse_g = m + math.log(np.exp(row - m).sum())
            out[g] = np.exp(row - lse_g) @ vc[h, A]
            lse[g] = lse_g
    return out, lse


# ------------------------------------------------- KV append, rollback ---

def unified_rows(is_verify: np.ndarray, k: int) -> np.ndarray:
    """Rows one unified iteration carries per request: the k+1 verify tokens
    of a verifying request, the one draft token of a drafting request
    [Unified batch scheduler, paper §4.2]."""
    return np.where(np.asarray(is_verify, bool), k + 1, 1).astype(np.int64)


def kv_append(k_pages: np.ndarray, v_pages: np.ndarray, block_table: np.ndarray,
              k_new: np.ndarray, v_new: np.ndarray, ctx_lens: np.ndarray, nrows: np.ndarray,
              page_size: int = 16) -> Tuple[np.ndarray, np.ndarray, bool]:
    """Write the current tokens' key and value rows into the paged cache
    [Dynamic KV-Cache management, paper §4.4: every decode step adds the KV
    of each request's new tokens; a verify carries k+1 tokens per request].

    Request r owns nrows[r] consecutive rows of k_new / v_new
    ([rows][Hkv][d], packed in request order): the tokens at positions
    ctx_lens[r] - nrows[r] .. ctx_lens[r] - 1.  Token j goes to page
    block_table[r][j // page_size], slot j % page_size, for every KV head.
    A row whose position is negative, beyond the block table's row, or
    whose page is outside the pool is skipped (and reported).
    Returns (new k_pages, new v_pages, any_skipped); the inputs are not
    modified.  Bit patterns are copied unchanged.
    """
    kp, vp = k_pages.copy(), v_pages.copy()
    num_pages = kp.shape[0]
    bt = np.asarray(block_table)
    skipped = False
    off = 0
    for r in range(len(ctx_lens)):
        n = int(nrows[r])
        for i in range(n):
            j = int(ctx_lens[r]) - n + i
            page = int(bt[r, j // page_size]) if 0 <= j < bt.shape[1] * page_size else -1
            if page < 0 or page >= num_pages:
                skipped = True
                continue
            kp[page, :, j % page_size, :] = k_new[off + i]
            vp[page, :, j % page_size, :] = v_new[off + i]
        off += n
    return kp, vp, skipped


def kv_rollback(ctx_lens: np.ndarray, sel_len: np.ndarray, is_verify: np.ndarray,
                accepted: np.ndarray, k: int) -> Tuple[np.ndarray, np.ndarray]:
    """Context after a verification [Delayed verification, paper §4.3: the
    verify phase decides which draft tokens are accepted; the rest are
    rejected].  A verifying request of context L (its k+1 verify tokens
    included: the last committed token and k drafts) that accepted a of its
    k drafts keeps L - k + a tokens; the KV of the rejected positions stays
    in the pages but lies past the context.  Selected tokens at or past the
    new length leave later draft sets: sel_len = min(sel_len, new length).
    Drafting requests are unchanged.  a is clamped to [0, k].
    Returns (new ctx_lens, new sel_len)."""
    isv = np.asarray(is_verify, bool)
    a = np.clip(np.asarray(accepted, np.int64), 0, k)
    ctx = np.asarray(ctx_lens, np.int64)
    new_ctx = np.where(isv, ctx - (k - a), ctx)
    new_sel = np.where(isv, np.minimum(np.asarray(sel_len, np.int64), new_ctx), np.asarray(sel_len, np.int64))
    return new_ctx, new_sel


# -------------------------------------------------------------- unified ---

def unified_step(q_rows: np.ndarray, k_pages: np.ndarray, v_pages: np.ndarray,
                 block_table: np.ndarray, ctx_lens: np.ndarray, is_verify: np.ndarray,
                 k: int, s: float, sm_scale: float, sel_in: List[np.ndarray],
                 sel_len_in: np.ndarray, page_size: int = 16,
                 requests: Sequence[int] = None):
    """One unified launch over a mixed batch [Unified batch scheduler, paper
    §4.2, Fig. 8]: requests of the verify bucket run verify attention and
    then the selection (which replaces their index sets); every other
    request runs one sparse draft step with its current index set.

    q_rows: float64 [rows][Hq][d] packed in request order (k+1 rows per
    verify request, 1 per draft request).
    Returns (out [rows][Hq][d], lse [rows][Hq], sel list, sel_len array)
    restricted to `requests` (all when None); rows of other requests are
    left as NaN.
    """
    B = len(ctx_lens)
    nrows = np.where(is_verify, k + 1, 1)
    offs = np.concatenate([[0], np.cumsum(nrows)])
    out = np.full(q_rows.shape, np.nan)
    lse = np.full(q_rows.shape[:2], np.nan)
    sel_out = list(sel_in)
    sel_len_out = np.array(sel_len_in, dtype=np.int64).copy()
    todo = range(B) if requests is None else requests
    hkv = k_pages.shape[1]
    for r in todo:
        L = int(ctx_lens[r])
        kc = gather_kv(k_pages, block_table[r], L, page_size)
        vc = gather_kv(v_pages, block_table[r], L, page_size)
        a, b = offs[r], offs[r + 1]
        if is_verify[r]:
            o, l, lg = verify_attention(q_rows[a:b], kc, vc, sm_scale)
            sel, _ = pillar_topk(lg, l, hkv, s)
            out[a:b], lse[a:b] = o, l
            sel_out[r] = sel
            sel_len_out[r] = L
        else:
            o, l = sparse_draft_attention(q_rows[a], kc, vc, sel_in[r],
                                          int(sel_len_in[r]), L, sm_scale)
            out[a], lse[a] = o, l
    return out, lse, sel_out, sel_len_out

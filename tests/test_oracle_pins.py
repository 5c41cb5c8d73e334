"""Pins of the CPU oracle against facts that do not come from the oracle.

Every function of oracle/sspec_ref.py is checked here against a library
routine (torch's scaled_dot_product_attention / logsumexp / softmax), a
closed form, an invariant, or exhaustive search on tiny inputs.  The cases
are chosen so that a dropped term, a flipped mask, a wrong head grouping, a
transposed operand or a wrong tie rule fails at least one of them.
"""

import itertools
import math

import numpy as np
import pytest
import torch

import oracle as O

pytestmark = pytest.mark.filterwarnings("ignore::UserWarning")


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _sdpa_decode(q, kc, vc, scale, n_vis):
    """torch SDPA in float64 with GQA; query i sees keys [0, n_vis[i])."""
    kp1, hq, d = q.shape
    hkv, L, _ = kc.shape
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]          # [1][Hq][k+1][d]
    kt = torch.from_numpy(kc)[None]                          # [1][Hkv][L][d]
    vt = torch.from_numpy(vc)[None]
    mask = torch.zeros(kp1, L, dtype=torch.bool)
    for i in range(kp1):
        mask[i, : n_vis[i]] = True
    o = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, attn_mask=mask, scale=scale, enable_gqa=(hq != hkv))
    G = hq // hkv
    kx = kt.repeat_interleave(G, dim=1)
    sc = scale * (qt @ kx.transpose(-1, -2))
    sc = sc.masked_fill(~mask, float("-inf"))
    lse = torch.logsumexp(sc, dim=-1)                        # [1][Hq][k+1]
    probs = torch.softmax(sc, dim=-1)
    return (o[0].permute(1, 0, 2).numpy(), lse[0].T.numpy(), probs[0].numpy())


# ------------------------------------------------------------- verify ---

@pytest.mark.parametrize("hq,hkv,k,L", [(4, 4, 0, 37), (4, 2, 3, 40), (6, 2, 4, 23), (8, 8, 2, 5)])
def test_verify_matches_torch_sdpa(hq, hkv, k, L):
    rng = np.random.default_rng(hq * 100 + k * 10 + L)
    d = 16
    q, kc, vc = _rand(rng, k + 1, hq, d), _rand(rng, hkv, L, d), _rand(rng, hkv, L, d)
    scale = float(np.float32(1 / math.sqrt(d)))
    out, lse, logits = O.verify_attention(q, kc, vc, scale)
    n_vis = [L - (k + 1) + i + 1 for i in range(k + 1)]
    o_ref, lse_ref, _ = _sdpa_decode(q, kc, vc, scale, n_vis)
    np.testing.assert_allclose(out, o_ref, atol=1e-12, rtol=1e-10)
    np.testing.assert_allclose(lse, lse_ref, atol=1e-12, rtol=1e-12)
    # dumped logits: finite exactly on the causal prefix of each query
    for i in range(k + 1):
        assert np.isfinite(logits[:, i, : n_vis[i]]).all()
        assert np.isneginf(logits[:, i, n_vis[i]:]).all()


def test_verify_closed_form_zero_keys():
    """All keys zero => all visible logits 0, LSE_i = ln(p_i + 1),
    O[i] = mean of V over [0, p_i] (p_i = L-k-1+i)."""
    rng = np.random.default_rng(3)
    hq, hkv, k, L, d = 6, 3, 4, 29, 8
    q = _rand(rng, k + 1, hq, d)
    kc = np.zeros((hkv, L, d))
    vc = _rand(rng, hkv, L, d)
    out, lse, logits = O.verify_attention(q, kc, vc, 0.125)
    G = hq // hkv
    for i in range(k + 1):
        p = L - k - 1 + i
        assert np.all(logits[:, i, : p + 1] == 0.0)
        np.testing.assert_allclose(lse[i], math.log(p + 1), rtol=0, atol=1e-13)
        for g in range(hq):
            np.testing.assert_allclose(out[i, g], vc[g // G, : p + 1].mean(0), atol=1e-13)


def test_verify_normalisation_invariant():
    """sum_j exp(logit - LSE) = 1 for every (head, query)."""
    rng = np.random.default_rng(5)
    q, kc, vc = _rand(rng, 9, 8, 32) * 3, _rand(rng, 4, 300, 32), _rand(rng, 4, 300, 32)
    _, lse, logits = O.verify_attention(q, kc, vc, 0.2)
    tot = np.exp(logits - lse.T[:, :, None]).sum(-1)
    np.testing.assert_allclose(tot, 1.0, atol=1e-12)


# ---------------------------------------------------------- selection ---

def test_scores_closed_form_zero_keys():
    """S[h, j] = (1/(k+1)) * sum_i [j <= p_i] / (p_i + 1) for all-zero keys."""
    rng = np.random.default_rng(7)
    hq, hkv, k, L, d = 8, 2, 5, 33, 8
    q, vc = _rand(rng, k + 1, hq, d), _rand(rng, hkv, L, d)
    _, lse, logits = O.verify_attention(q, np.zeros((hkv, L, d)), vc, 0.3)
    S = O.pillar_scores(logits, lse, hkv)
    expect = np.zeros(L)
    for i in range(k + 1):
        p = L - k - 1 + i
        expect[: p + 1] += 1.0 / (p + 1)
    expect /= k + 1
    for h in range(hkv):
        np.testing.assert_allclose(S[h], expect, rtol=1e-13, atol=0)


def test_scores_one_hot_gqa_average():
    """Each (query head g, query i) puts all its mass on one target token
    t(g, i); then S[h, j] is the fraction of the G*(k+1) rows of group h
    that target j.  Fails for a wrong head->group map or a wrong mean."""
    hq, hkv, k = 6, 2, 2
    G = hq // hkv
    L = 12
    d = L
    big = 80.0
    kc = np.zeros((hkv, L, d))
    for h in range(hkv):
        kc[h] = np.eye(L) * big
    # targets inside the causal window of each query (p_i = L-k-1+i >= 9)
    targets = np.array([[(3 * g + 2 * i + g // G) % 9 for i in range(k + 1)] for g in range(hq)])
    q = np.zeros((k + 1, hq, d))
    for g in range(hq):
        for i in range(k + 1):
            q[i, g, targets[g, i]] = 1.0
    _, lse, logits = O.verify_attention(q, kc, np.zeros((hkv, L, d)), 1.0)
    S = O.pillar_scores(logits, lse, hkv)
    for h in range(hkv):
        cnt = np.zeros(L)
        for g in range(h * G, (h + 1) * G):
            for i in range(k + 1):
                cnt[targets[g, i]] += 1
        np.testing.assert_allclose(S[h], cnt / (G * (k + 1)), atol=1e-20)


def test_scores_match_torch_softmax():
    """Random inputs: the scores recovered from the logit + LSE dump equal
    the group/query mean of torch's softmax attention weights."""
    rng = np.random.default_rng(11)
    hq, hkv, k, L, d = 8, 4, 3, 50, 16
    q, kc, vc = _rand(rng, k + 1, hq, d) * 2, _rand(rng, hkv, L, d), _rand(rng, hkv, L, d)
    _, lse, logits = O.verify_attention(q, kc, vc, 0.25)
    n_vis = [L - (k + 1) + i + 1 for i in range(k + 1)]
    _, _, probs = _sdpa_decode(q, kc, vc, 0.25, n_vis)       # [Hq][k+1][L]
    S = O.pillar_scores(logits, lse, hkv)
    G = hq // hkv
    ref = probs.reshape(hkv, G * (k + 1), L).mean(1)
    np.testing.assert_allclose(S, ref, rtol=1e-11, atol=1e-15)


def test_topk_exhaustive_search():
    """K largest with lowest-index tie-break == the maximum-sum K-subset
    that is lexicographically smallest (integer scores, so sums are exact)."""
    rng = np.random.default_rng(13)
    for trial in range(300):
        L = int(rng.integers(1, 11))
        K = int(rng.integers(1, min(L, 4) + 1))
        sc = rng.integers(0, 4, size=L).astype(np.float64)   # many ties
        best = None
        for sub in itertools.combinations(range(L), K):
            key = (-sc[list(sub)].sum(), sub)
            if best is None or key < best:
                best = key
        got = O.topk_lowest_index(sc, K)
        assert tuple(got.tolist()) == best[1], (sc, K, got, best)


def test_topk_flat_scores_take_lowest_indices():
    """All-zero keys: S is constant on [0, L-k-1] and smaller after, so the
    selection is exactly [0, K)."""
    rng = np.random.default_rng(17)
    hq, hkv, k, L, d = 4, 2, 8, 200, 8
    q, vc = _rand(rng, k + 1, hq, d), _rand(rng, hkv, L, d)
    _, lse, logits = O.verify_attention(q, np.zeros((hkv, L, d)), vc, 0.3)
    sel, K = O.pillar_topk(logits, lse, hkv, 0.05)
    assert K == 10
    for h in range(hkv):
        assert sel[h].tolist() == list(range(K))


def test_topk_planted_pillars():
    """Strongly separated planted tokens are selected exactly."""
    rng = np.random.default_rng(19)
    hq, hkv, k, L, d = 8, 2, 8, 400, 32
    G = hq // hkv
    kc, vc = _rand(rng, hkv, L, d), _rand(rng, hkv, L, d)
    q = _rand(rng, k + 1, hq, d)
    planted = []
    for h in range(hkv):
        u = _rand(rng, d)
        u /= np.linalg.norm(u)
        pos = np.sort(rng.choice(L - k - 1, size=20, replace=False))
        planted.append(pos)
        kc[h, pos] += 8 * u
        q[:, h * G:(h + 1) * G] += 4 * math.sqrt(d) * u
    _, lse, logits = O.verify_attention(q, kc, vc, 1 / math.sqrt(d))
    sel, K = O.pillar_topk(logits, lse, hkv, 20 / L)
    assert K == 20
    for h in range(hkv):
        assert sel[h].tolist() == planted[h].tolist()


def _golden_counts():
    rows = []
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "select_counts.txt")
    for line in open(path):
        line = line.split("#")[0].strip()
        if line:
            L, s, K = line.split()
            rows.append((int(L), float(s), int(K)))
    return rows


@pytest.mark.parametrize("L,s,K", _golden_counts())
def test_select_count_golden(L, s, K):
    assert O.select_count(L, s) == K


def test_selection_invariants_random():
    rng = np.random.default_rng(23)
    for _ in range(20):
        hq, hkv, k = 8, 4, int(rng.integers(0, 6))
        L = int(rng.integers(k + 1, 120))
        s = float(rng.choice([0.01, 0.05, 0.1, 0.37, 1.0]))
        q, kc, vc = _rand(rng, k + 1, hq, 8), _rand(rng, hkv, L, 8), _rand(rng, hkv, L, 8)
        _, lse, logits = O.verify_attention(q, kc, vc, 0.4)
        sel, K = O.pillar_topk(logits, lse, hkv, s)
        assert K == min(L, math.ceil(s * L)) and sel.shape == (hkv, K)
        for h in range(hkv):
            assert np.all(np.diff(sel[h]) > 0) and sel[h].min() >= 0 and sel[h].max() < L


# -------------------------------------------------------------- draft ---

def test_draft_full_selection_is_full_attention():
    """s = 1.0 selects every token, and with the appended tail the draft
    query attends to all of [0, ctx_len): equal to torch SDPA."""
    rng = np.random.default_rng(29)
    hq, hkv, d, sel_len, ctx = 8, 2, 16, 60, 66
    kc, vc = _rand(rng, hkv, ctx, d), _rand(rng, hkv, ctx, d)
    qv = _rand(rng, 4, hq, d)
    _, lse, logits = O.verify_attention(qv, kc[:, :sel_len], vc[:, :sel_len], 0.25)
    sel, K = O.pillar_topk(logits, lse, hkv, 1.0)
    assert K == sel_len
    qd = _rand(rng, hq, d)
    out, l = O.sparse_draft_attention(qd, kc, vc, sel, sel_len, ctx, 0.25)
    o_ref, lse_ref, _ = _sdpa_decode(qd[None], kc, vc, 0.25, [ctx])
    np.testing.assert_allclose(out, o_ref[0], atol=1e-12)
    np.testing.assert_allclose(l, lse_ref[0], atol=1e-12)


def test_draft_zero_keys_uniform_over_token_set():
    """All-zero keys: O = mean of V over exactly the selected tokens that are
    < ctx_len plus the tail [sel_len, ctx_len); LSE = ln(size)."""
    rng = np.random.default_rng(31)
    hq, hkv, d = 4, 2, 8
    for sel_len, ctx in [(50, 55), (50, 50), (50, 41)]:
        kc, vc = np.zeros((hkv, 64, d)), _rand(rng, hkv, 64, d)
        sel = [np.array([0, 7, 8, 30, 44, 49]), np.array([3, 40, 45, 46])]
        out, lse = O.sparse_draft_attention(_rand(rng, hq, d), kc, vc, sel, sel_len, ctx, 0.5)
        for g in range(hq):
            h = g // (hq // hkv)
            toks = sorted({int(j) for j in sel[h] if j < min(sel_len, ctx)} |
                          set(range(sel_len, max(sel_len, ctx))))
            np.testing.assert_allclose(out[g], vc[h, toks].mean(0), atol=1e-13)
            np.testing.assert_allclose(lse[g], math.log(len(toks)), atol=1e-13)


# ------------------------------------------------------ paging, unified ---

def _paged(rng, hkv, L, d, page, extra=5):
    npg = -(-L // page)
    total = npg + extra
    perm = rng.permutation(total)[:npg]
    kf = rng.standard_normal((L, hkv, d)).astype(np.float32)
    bits = (kf.view(np.uint32) >> 16).astype(np.uint16)       # truncated to bf16 bits
    pages = np.zeros((total, hkv, page, d), np.uint16)
    for p in range(npg):
        n = min(page, L - p * page)
        pages[perm[p], :, :n, :] = bits[p * page: p * page + n].transpose(1, 0, 2)
    return pages, perm, bits


def test_gather_follows_block_table_and_permutation_invariance():
    rng = np.random.default_rng(37)
    hkv, L, d, page = 3, 45, 8, 16
    pages, bt, bits = _paged(rng, hkv, L, d, page)
    kc = O.gather_kv(pages, bt, L, page)
    expect = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64).transpose(1, 0, 2)
    assert np.array_equal(kc, expect)
    # move the physical pages around, rewrite the table: bit-identical result
    newpos = rng.permutation(pages.shape[0])
    pages2 = np.empty_like(pages)
    pages2[newpos] = pages
    assert np.array_equal(O.gather_kv(pages2, newpos[bt], L, page), kc)


def test_unified_is_per_request_application():
    rng = np.random.default_rng(41)
    hq, hkv, d, page, k, s = 4, 2, 8, 16, 3, 0.2
    Ls = [40, 33, 57]
    is_v = np.array([True, False, False])
    kp, bt, vp = [], [], []
    total = 0
    pages_k = np.zeros((0, hkv, page, d), np.uint16)
    pages_v = np.zeros((0, hkv, page, d), np.uint16)
    bts = np.zeros((3, 8), np.int64)
    for r, L in enumerate(Ls):
        pk, perm, _ = _paged(rng, hkv, L, d, page, extra=0)
        pv, _, _ = _paged(rng, hkv, L, d, page, extra=0)
        pv = pv[np.argsort(perm)][perm]  # same physical slots as keys
        bts[r, : len(perm)] = perm + pages_k.shape[0]
        pages_k = np.concatenate([pages_k, pk])
        pages_v = np.concatenate([pages_v, pv])
    rows = np.where(is_v, k + 1, 1)
    q = _rand(rng, rows.sum(), hq, d)
    sel_in = [None, [np.array([1, 5, 9]), np.array([0, 2])], [np.array([3]), np.array([4, 6])]]
    sel_len = np.array([0, 30, 50])
    out, lse, sel, sl = O.unified_step(q, pages_k, pages_v, bts, np.array(Ls), is_v, k, s, 0.35,
                                       sel_in, sel_len, page)
    kc0 = O.gather_kv(pages_k, bts[0], Ls[0], page)
    vc0 = O.gather_kv(pages_v, bts[0], Ls[0], page)
    o0, l0, lg0 = O.verify_attention(q[: k + 1], kc0, vc0, 0.35)
    s0, _ = O.pillar_topk(lg0, l0, hkv, s)
    np.testing.assert_array_equal(out[: k + 1], o0)
    np.testing.assert_array_equal(sel[0], s0)
    assert sl[0] == Ls[0] and sl[1] == 30 and sl[2] == 50
    for r, row in [(1, k + 1), (2, k + 2)]:
        kc = O.gather_kv(pages_k, bts[r], Ls[r], page)
        vc = O.gather_kv(pages_v, bts[r], Ls[r], page)
        o, l = O.sparse_draft_attention(q[row], kc, vc, sel_in[r], sel_len[r], Ls[r], 0.35)
        np.testing.assert_array_equal(out[row], o)
        np.testing.assert_array_equal(lse[row], l)


def test_bf16_widening_matches_torch():
    """bf16_to_f64 against torch's own bfloat16 -> float64 conversion, over
    every one of the 65536 bit patterns (NaNs compared as NaN)."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    got = O.bf16_to_f64(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zeros and infinities keep their sign
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


# ------------------------------------------------------- KV append/rollback ---

def _pool(rng, num_pages, hkv, d, page=16):
    return rng.integers(0, 1 << 16, size=(num_pages, hkv, page, d), dtype=np.uint64).astype(np.uint16)


def test_kv_append_contiguous_table_read_back_by_reshape():
    """With request r owning pages [r*P, (r+1)*P) in order, the pool viewed
    as tokens [r][P*16] (a plain transpose + reshape) must hold the new rows
    at positions ctx-n .. ctx-1 of each request, and every other token must
    keep its bits."""
    rng = np.random.default_rng(11)
    B, P, hkv, d, k = 4, 5, 3, 8, 3
    kp, vp = _pool(rng, B * P, hkv, d), _pool(rng, B * P, hkv, d)
    bt = np.arange(B * P).reshape(B, P)
    ctx = np.array([20, 4, 80, 37])
    isv = np.array([True, True, False, False])
    nrows = O.unified_rows(isv, k)
    assert nrows.tolist() == [4, 4, 1, 1]
    rows = int(nrows.sum())
    k_new, v_new = _pool(rng, rows, hkv, d, page=1)[:, :, 0, :], _pool(rng, rows, hkv, d, page=1)[:, :, 0, :]
    k_new = np.ascontiguousarray(k_new)
    v_new = np.ascontiguousarray(v_new)
    kp2, vp2, skipped = O.kv_append(kp, vp, bt, k_new, v_new, ctx, nrows)
    assert not skipped
    tok = lambda pool: pool.reshape(B, P, hkv, 16, d).transpose(0, 1, 3, 2, 4).reshape(B, P * 16, hkv, d)
    before_k, after_k, after_v = tok(kp), tok(kp2), tok(vp2)
    off = np.concatenate([[0], np.cumsum(nrows)])
    changed = np.zeros((B, P * 16), bool)
    for r in range(B):
        lo = ctx[r] - nrows[r]
        assert np.array_equal(after_k[r, lo: ctx[r]], k_new[off[r]: off[r + 1]])
        assert np.array_equal(after_v[r, lo: ctx[r]], v_new[off[r]: off[r + 1]])
        changed[r, lo: ctx[r]] = True
    assert np.array_equal(after_k[~changed], before_k[~changed])
    assert np.array_equal(tok(vp)[~changed], after_v[~changed])
    assert np.array_equal(kp, tok(kp).reshape(B, P, 16, hkv, d).transpose(0, 1, 3, 2, 4).reshape(kp.shape))


def test_kv_append_paging_invariance_and_gather():
    """Permuting the physical pages (and the block table with them) permutes
    the result the same way; gather_kv then reads the new rows back as each
    request's last tokens."""
    rng = np.random.default_rng(12)
    B, P, hkv, d = 3, 4, 2, 8
    kp, vp = _pool(rng, B * P, hkv, d), _pool(rng, B * P, hkv, d)
    bt = np.arange(B * P).reshape(B, P)
    perm = rng.permutation(B * P)          # logical page p -> physical perm[p]
    kq, vq = np.empty_like(kp), np.empty_like(vp)
    kq[perm], vq[perm] = kp, vp
    btq = perm[bt]
    ctx = np.array([33, 64, 17])
    nrows = np.array([3, 1, 2])
    k_new = rng.integers(0, 1 << 16, size=(6, hkv, d), dtype=np.uint64).astype(np.uint16)
    v_new = rng.integers(0, 1 << 16, size=(6, hkv, d), dtype=np.uint64).astype(np.uint16)
    a_k, a_v, _ = O.kv_append(kp, vp, bt, k_new, v_new, ctx, nrows)
    b_k, b_v, _ = O.kv_append(kq, vq, btq, k_new, v_new, ctx, nrows)
    assert np.array_equal(b_k[perm], a_k) and np.array_equal(b_v[perm], a_v)
    off = np.concatenate([[0], np.cumsum(nrows)])
    for r in range(B):
        got = O.gather_kv(b_k, btq[r], int(ctx[r]), 16)            # [Hkv][ctx][d]
        want = O.bf16_to_f64(k_new[off[r]: off[r + 1]]).transpose(1, 0, 2)
        assert np.array_equal(got[:, ctx[r] - nrows[r]:], want, equal_nan=True)   # random bits hold NaNs


def test_kv_append_skips_bad_rows():
    """A position past the block table's row or a page outside the pool is
    skipped and reported; the other rows are written."""
    rng = np.random.default_rng(13)
    kp, vp = _pool(rng, 4, 1, 8), _pool(rng, 4, 1, 8)
    bt = np.array([[0, 1], [2, 9]])       # request 1's second page is outside the pool
    k_new = rng.integers(0, 1 << 16, size=(3, 1, 8), dtype=np.uint64).astype(np.uint16)
    a_k, _, skipped = O.kv_append(kp, vp, bt, k_new, k_new, np.array([33, 20]), np.array([2, 1]))
    assert skipped
    assert np.array_equal(a_k[2], kp[2]) and np.array_equal(a_k[3], kp[3])   # request 1 untouched
    assert np.array_equal(a_k[1, 0, 15], k_new[0, 0])                        # position 31: page 1 slot 15
    assert np.array_equal(a_k[0], kp[0])                                     # position 32 is past 2 pages


def test_kv_rollback_closed_forms():
    """All k drafts accepted: context unchanged; none: k tokens dropped; the
    selection length is cut to the new context; drafting requests and
    out-of-range counts (clamped) behave as stated."""
    k = 8
    ctx = np.array([1000, 1000, 1000, 500, 777])
    sel_len = np.array([1000, 1000, 995, 480, 770])
    isv = np.array([True, True, True, False, True])
    acc = np.array([8, 0, 3, 5, 12])
    new_ctx, new_sel = O.kv_rollback(ctx, sel_len, isv, acc, k)
    assert new_ctx.tolist() == [1000, 992, 995, 500, 777]
    assert new_sel.tolist() == [1000, 992, 995, 480, 770]
    new_ctx, _ = O.kv_rollback(ctx, sel_len, isv, np.array([-4, 0, 0, 0, 0]), k)
    assert new_ctx[0] == 992

"""Host checks of the seeded input generator (no GPU)."""

import math

import numpy as np
import torch

from sspec_workload import (assign_buckets_least_loaded, context_lengths, cycle_state,
                            make_workload, pack_rows, workload_spec)


def test_seed_reproducible_and_pages_permuted():
    spec = workload_spec(1, batch=3)
    a = make_workload(spec, seed=5, lengths=[100, 37, 64])
    b = make_workload(spec, seed=5, lengths=[100, 37, 64])
    c = make_workload(spec, seed=6, lengths=[100, 37, 64])
    assert torch.equal(a.k_pages.view(torch.int16), b.k_pages.view(torch.int16))
    assert torch.equal(a.qbank.view(torch.int16), b.qbank.view(torch.int16))
    assert not torch.equal(a.k_pages.view(torch.int16), c.k_pages.view(torch.int16))
    used = []
    for r in range(a.batch):
        npg = -(-int(a.caps[r]) // a.page_size)
        used += a.block_table[r, :npg].tolist()
    assert sorted(used) == list(range(a.num_pages))          # every page used once
    assert used != sorted(used)                               # not contiguous


def test_pillar_count_and_range():
    spec = workload_spec(0)
    w = make_workload(spec, seed=0)
    assert w.verify_lens.tolist() == [2048]
    pos = w.pillar_pos[0]
    assert pos.shape == (8, round(0.05 * 2048))
    for h in range(8):
        assert len(set(pos[h].tolist())) == pos.shape[1] and pos[h].max() < 2048


def test_least_loaded_buckets():
    b = assign_buckets_least_loaded(128, 9)
    cnt = np.bincount(b, minlength=9)
    assert cnt.max() - cnt.min() <= 1 and cnt.sum() == 128
    assert cnt.tolist() == [15, 15] + [14] * 7


def test_lognormal_lengths_statistics():
    rng = np.random.default_rng(0)
    L = context_lengths(("lognormal", 12000.0, 7600.0, 1024, 32768), 200000, rng)
    assert L.min() >= 1024 and L.max() <= 32768
    # clipping trims the mean a little below 12000 (about 11.8K)
    assert 11600 < L.mean() < 12000
    clip_hi = (L == 32768).mean()
    assert 0.015 < clip_hi < 0.03


def test_cycle_state_rows():
    spec = workload_spec(1, batch=5, k=2)
    w = make_workload(spec, seed=1, lengths=[20, 21, 22, 23, 24])
    for t in range(3):
        vb, isv, ctx, step = cycle_state(w, t)
        assert (isv == (w.bucket_ids == vb)).all()
        assert (ctx[isv] == w.verify_lens[isv]).all()
        assert ((ctx[~isv] - w.verify_lens[~isv]) >= 1).all()
        assert ((ctx[~isv] - w.verify_lens[~isv]) <= w.k).all()
        q = pack_rows(w, isv, step)
        assert q.shape[0] == int(np.where(isv, w.k + 1, 1).sum())

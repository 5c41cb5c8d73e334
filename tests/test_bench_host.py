"""Host logic of bench.py: the one-GPU guard, the algorithmic byte model
and the layer-cycled launch order, with the library replaced by a recorder
(no GPU)."""

import subprocess
import sys

import numpy as np
import pytest
import torch

import bench
from sspec_workload import make_workload, workload_spec


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU only" in r.stderr and r.stdout == ""


def test_algorithmic_bytes_hand_worked():
    # head_dim 128, 2 query / 1 KV head, k = 1, s = 0.05.
    # request 0 verifies at L = 32 (K = ceil(1.6) = 2 selected):
    #   K+V 32*128*2*2 = 16384, dump written and read 2*32*2*2*4 = 1024,
    #   indices 2*4 = 8, Q read + O written 2*2*2*128*2 = 2048, LSE 2*2*4 = 16
    # request 1 drafts with 3 selected tokens at step 1 (4 rows read):
    #   K+V 4*128*2*2 = 2048, indices 3*4 = 12, Q + O 2*2*128*2 = 1024, LSE 8
    got = bench.algorithmic_bytes(np.array([32, 100]), np.array([True, False]), np.array([0, 1]),
                                  np.array([0, 3]), k=1, s=0.05, hq=2, hkv=1)
    assert got == (16384 + 1024 + 8 + 2048 + 16) + (2048 + 12 + 1024 + 8)


class _Recorder:
    """Stands in for the binding: records what each unified launch reads."""

    def __init__(self):
        self.calls = []

    class PagedKV:
        def __init__(self, k, v, bt):
            self.k_pages, self.v_pages, self.block_table = k, v, bt

    @staticmethod
    def unified_workspace_size(*a):
        return 4096

    @staticmethod
    def workspace(n, dev):
        return torch.zeros(n, dtype=torch.uint8)

    @staticmethod
    def read_device_error(ws):
        return 0

    def unified_attn(self, kv, q, ctx, bk, vb, B, mv, mc, hq, k, s, sc, sel, ss, cnt, sl, out, lse, ws):
        self.calls.append((kv.k_pages.data_ptr(), q.data_ptr(), sel.data_ptr(), out.data_ptr(), int(vb)))
        cnt.fill_(5)


def test_layer_cycled_launch_order(monkeypatch):
    monkeypatch.setattr(torch.cuda, "synchronize", lambda: None)
    spec = workload_spec(1, batch=6, lengths=("uniform", 300, 900))
    w = make_workload(spec, seed=1, device="cpu")
    rec = _Recorder()
    layers = 3
    h = bench.LayerHarness(rec, w, w.s, layers, dev="cpu")
    h.setup_cycle()
    kp1 = w.k + 1
    assert len(rec.calls) == kp1 * layers
    for t, (kp, q, sel, out, vb) in enumerate(rec.calls):
        P, i = h.per[t % layers], (t // layers) % kp1   # every layer of a step, then the next step
        assert kp == P["kv"].k_pages.data_ptr() and q == P["qs"][i].data_ptr()
        assert sel == P["sel"].data_ptr() and out == P["outs"][i].data_ptr()
        assert vb == int(h.cycles[i][0])
    # each layer owns its pools (same values, its own memory) and its state
    assert len({c[0] for c in rec.calls}) == layers and len({c[2] for c in rec.calls}) == layers
    for P in h.per[1:]:
        assert torch.equal(P["kv"].k_pages, w.k_pages) and P["kv"].k_pages.data_ptr() != w.k_pages.data_ptr()
    # bytes and queries of `layers` launches per step equal `layers` times the one-layer figures
    one = bench.Harness(rec, w, w.s, "cpu")
    one.cnt.fill_(5)
    b1, q1 = one.bytes_and_queries(kp1)
    bl, ql = h.bytes_and_queries(kp1 * layers)
    assert (bl, ql) == (layers * b1, layers * q1)

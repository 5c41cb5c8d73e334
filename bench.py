"""Benchmark of the SparseSpec attention hot path on one MI355X.

Default (--bench unified): the Qwen3-8B attention shape (32 query / 8 KV
heads, head_dim 128, bf16), batch 128, verify-time contexts lognormal with
mean 12000 and sd 7600 clipped to [1024, 32768], k = 8, s = 0.05, page 16,
requests spread over k+1 buckets by least-loaded assignment.  One step is
one unified launch (one attention layer): the requests of one bucket verify
(k+1 queries, full attention, logit+LSE dump, PillarAttn Top-K) and all the
others run one sparse draft step.  Timed steps rotate the verify bucket, so
every full cycle of k+1 steps verifies each request once.  Prints ONE JSON
line: queries/s (one query = one query token of one request across all
heads), the unified kernel's algorithmic HBM bandwidth against the 8 TB/s
peak (and against a device copy measured in the same run), and the CPU
oracle timed on a bounded sample on this host.

Other modes (each prints its own JSON line per measured point):
  --bench separate   the same rotation through three launches per step
                     (sspec_verify_attn -> sspec_pillar_topk ->
                     sspec_sparse_draft_attn on one stream), next to the
                     unified launch on the same inputs;
  --bench naive      the fused launch vs the naive-batching launch
                     (sspec_unified_attn_naive: every item in the verify's
                     tile shape) vs the separate launches, same steps;
  --bench offload    the unified rotation with the KV offload engine moving
                     a cold pool's pages to pinned host memory and back on
                     a side stream, at several rates: step-time overhead;
  --bench loop       a decode loop driven by the native scheduler (36
                     layers per iteration), synchronous vs delayed
                     verification;
  --bench layers     the unified rotation cycling over the KV caches of many
                     attention layers (--kv-layers, as many as fit), one
                     decode step through every layer after another;
  --bench kv_append  sspec_kv_append of each step's rows (k+1 per verifying
                     request, 1 per drafting one);
  --bench sweep      the long-context sweep: batch 32, contexts 64K and
                     128K, k in {4, 8, 16}, s in {0.01, 0.05, 0.1, 1.0},
                     unified vs separate, and at s = 1 a sampled draft
                     checked against plain full attention (torch, fp32).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
METRIC = "unified attn queries/s + achieved HBM GB/s (% of peak), Qwen3-8B shape, B=128"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sparse_self_speculative_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(verify_lens, isv, step, sel_count, k, s, hq, hkv, d=128):
    """Bytes the method must move in one unified launch (one layer):
    verify item: K+V of its L tokens, the logit dump written and read back,
      the selected indices written, Q read, O written, LSE written;
    draft item: K+V rows of its selected tokens plus the appended tail, the
      index reads, Q read, O and LSE written."""
    total = 0
    for r in range(len(verify_lens)):
        L = int(verify_lens[r])
        if isv[r]:
            K = min(L, math.ceil(s * L))
            total += L * hkv * d * 2 * 2
            total += 2 * L * hq * (k + 1) * 4
            total += hkv * K * 4
            total += 2 * (k + 1) * hq * d * 2 + hq * (k + 1) * 4
        else:
            n = int(sel_count[r]) + int(step[r])
            total += n * hkv * d * 2 * 2 + int(sel_count[r]) * hkv * 4 + 2 * hq * d * 2 + hq * 4
    return total


def cpu_baseline(w, kp, vp, bt, cyc, budget_s: float):
    """Time the CPU oracle on a bounded sample of one launch's requests:
    verify + selection for verifying requests, one sparse draft step for
    drafting ones, in the launch's 1:8 mix, until budget_s of CPU time."""
    import oracle as O
    from sspec_workload import to_numpy_bf16
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
    vb, isv, ctx, step = cyc
    k, s, hkv = w.k, w.s, w.num_kv_heads
    q64 = O.bf16_to_f64(to_numpy_bf16(w.qbank))
    rng = np.random.default_rng(0)
    vids = [int(x) for x in rng.permutation(np.nonzero(isv)[0])[:4]]
    dids = [int(x) for x in rng.permutation(np.nonzero(~isv)[0])[:32]]
    # a draft's cost depends on how many tokens it reads, not which: each
    # sampled draft gets a random ascending set of ceil(s*L) tokens per head
    sels = {}
    for r in dids:
        Lv = int(w.verify_lens[r])
        K = O.select_count(Lv, s)
        sels[r] = [np.sort(rng.choice(Lv, K, replace=False)) for _ in range(hkv)]
    queries, spent, nv, nd, i = 0, 0.0, 0, 0, 0
    while spent < budget_s:
        r = vids[i % len(vids)]
        t0 = time.perf_counter()
        kc = O.gather_kv(kp, bt[r], int(ctx[r]), 16)
        vc = O.gather_kv(vp, bt[r], int(ctx[r]), 16)
        _, l, lg = O.verify_attention(q64[r, : k + 1], kc, vc, w.sm_scale)
        O.pillar_topk(lg, l, hkv, s)
        spent += time.perf_counter() - t0
        queries += k + 1
        nv += 1
        for j in range(8):
            r = dids[(8 * i + j) % len(dids)]
            t0 = time.perf_counter()
            kc = O.gather_kv(kp, bt[r], int(ctx[r]), 16)
            vc = O.gather_kv(vp, bt[r], int(ctx[r]), 16)
            O.sparse_draft_attention(q64[r, k + int(step[r])], kc, vc, sels[r],
                                     int(w.verify_lens[r]), int(ctx[r]), w.sm_scale)
            spent += time.perf_counter() - t0
            queries += 1
            nd += 1
        i += 1
    return {"value": queries / spent, "unit": "queries/s", "cores": int(blas_threads),
            "kind": "oracle",
            "sample": f"{nv} verify+select and {nd} draft calls (1:8 mix) on 4 verifying and 32 "
                      f"drafting requests of one launch of the same workload, float64 numpy "
                      f"oracle incl. its paged-KV gather, {spent:.1f} s timed; draft token sets random of size ceil(s*L); "
                      f"BLAS threads {blas_threads}, host cores {len(os.sched_getaffinity(0))}"}


class Harness:
    """One workload's unified launch sequence (and the same steps through the
    separate entry points) on the device."""

    def __init__(self, S, w, s, dev="cuda"):
        import torch
        from sspec_workload import cycle_state, pack_rows
        self.torch, self.S, self.w, self.s, self.dev = torch, S, w, s, dev
        B, hq, hkv, k = w.batch, w.num_q_heads, w.num_kv_heads, w.k
        self.kp1 = kp1 = k + 1
        self.max_ctx = int(w.caps.max())
        self.sel_stride = math.ceil(s * self.max_ctx)
        self.max_verify = int(np.bincount(w.bucket_ids, minlength=kp1).max())
        self.kv = S.PagedKV(w.k_pages, w.v_pages, w.block_table)
        self.ws = S.workspace(S.unified_workspace_size(B, self.max_verify, self.max_ctx, hq, hkv, k), dev)
        self.sel = torch.zeros(B, hkv, self.sel_stride, dtype=torch.int32, device=dev)
        self.cnt = torch.zeros(B, dtype=torch.int32, device=dev)
        self.sl = torch.from_numpy(w.verify_lens.astype(np.int32)).to(dev)
        self.bk = torch.from_numpy(w.bucket_ids).to(dev)
        self.cycles = [cycle_state(w, t) for t in range(kp1)]
        self.qs = [pack_rows(w, c[1], c[3], dev) for c in self.cycles]
        self.ctxs = [torch.from_numpy(c[2].astype(np.int32)).to(dev) for c in self.cycles]
        self.outs = [torch.empty_like(q) for q in self.qs]
        self.lses = [torch.empty(q.shape[0], hq, dtype=torch.float32, device=dev) for q in self.qs]
        self._sep = None

    def launch(self, t):
        w, i = self.w, t % self.kp1
        self.S.unified_attn(self.kv, self.qs[i], self.ctxs[i], self.bk, self.cycles[i][0], w.batch,
                            self.max_verify, self.max_ctx, w.num_q_heads, w.k, self.s, w.sm_scale, self.sel,
                            self.sel_stride, self.cnt, self.sl, self.outs[i], self.lses[i], self.ws)

    def launch_naive(self, t):
        """The same step through the naive-batching launch (one tile shape for
        every item), on its own workspace and selection state."""
        w, i = self.w, t % self.kp1
        if not hasattr(self, "_naive"):
            self._naive = (self.S.workspace(self.ws.numel(), self.dev), self.sel.clone(), self.cnt.clone(),
                           self.sl.clone(), [torch_empty_like(o) for o in self.outs],
                           [torch_empty_like(x) for x in self.lses])
        ws, sel, cnt, sl, outs, lses = self._naive
        self.S.unified_attn_naive(self.kv, self.qs[i], self.ctxs[i], self.bk, self.cycles[i][0], w.batch,
                                  self.max_verify, self.max_ctx, w.num_q_heads, w.k, self.s, w.sm_scale, sel,
                                  self.sel_stride, cnt, sl, outs[i], lses[i], ws)

    def setup_cycle(self):
        for t in range(self.kp1):   # every request verifies once: every draft holds a selection
            self.launch(t)
        self.torch.cuda.synchronize()
        flags = self.S.read_device_error(self.ws)
        if flags:
            raise RuntimeError(f"device error flags 0x{flags:x} in the set-up cycle")

    # ---- the same steps through the three separate entry points
    def _separate_state(self):
        if self._sep is not None:
            return self._sep
        torch, S, w = self.torch, self.S, self.w
        hq, hkv, k, kp1 = w.num_q_heads, w.num_kv_heads, w.k, self.kp1
        lstride = -(-self.max_ctx // 16) * 16
        st = dict(lstride=lstride, steps=[])
        nv_max, nd_max = 0, 0
        for i, (vb, isv, ctx, step) in enumerate(self.cycles):
            off = np.concatenate([[0], np.cumsum(np.where(isv, kp1, 1))])
            vid, did = np.nonzero(isv)[0], np.nonzero(~isv)[0]
            q = self.qs[i]
            d = dict(nv=len(vid), nd=len(did))
            if len(vid):
                d["qv"] = torch.stack([q[off[r]: off[r] + kp1] for r in vid]).contiguous()
                d["seq_v"] = torch.from_numpy(vid.astype(np.int32)).to(self.dev)
                d["out_v"] = torch.empty_like(d["qv"])
                d["lse_v"] = torch.empty(len(vid), kp1, hq, dtype=torch.float32, device=self.dev)
            if len(did):
                d["qd"] = torch.stack([q[off[r]] for r in did]).contiguous()
                d["seq_d"] = torch.from_numpy(did.astype(np.int32)).to(self.dev)
                d["out_d"] = torch.empty_like(d["qd"])
                d["lse_d"] = torch.empty(len(did), hq, dtype=torch.float32, device=self.dev)
            nv_max, nd_max = max(nv_max, len(vid)), max(nd_max, len(did))
            st["steps"].append(d)
        mp = S.dump_pitch(hq, hkv, k)
        st["logits"] = torch.empty(max(nv_max, 1), hkv, lstride // 16, mp, 16, dtype=torch.float32, device=self.dev)
        st["wsv"] = S.workspace(S.verify_workspace_size(max(nv_max, 1), self.max_ctx, hq, hkv, k), self.dev)
        st["wst"] = S.workspace(S.pillar_topk_workspace_size(max(nv_max, 1), self.max_ctx, hkv), self.dev)
        st["wsd"] = S.workspace(S.draft_workspace_size(max(nd_max, 1), self.max_ctx, hq, hkv), self.dev)
        # the separate path keeps its own selection state, started from the unified one
        st["sel"], st["cnt"], st["sl"] = self.sel.clone(), self.cnt.clone(), self.sl.clone()
        self._sep = st
        return st

    def launch_separate(self, t, marks=None):
        """verify -> pillar_topk -> draft for step t; `marks` (optional list of
        4 events) are recorded around the three launches."""
        S, w = self.S, self.w
        st = self._separate_state()
        i = t % self.kp1
        d = st["steps"][i]
        hq, hkv, k = w.num_q_heads, w.num_kv_heads, w.k
        stream = self.torch.cuda.current_stream()
        if marks:
            marks[0].record(stream)
        if d["nv"]:
            S.verify_attn(self.kv, d["qv"], d["seq_v"], self.ctxs[i], d["nv"], self.max_ctx, hq, k, w.sm_scale,
                          d["out_v"], d["lse_v"], st["logits"], st["lstride"], st["wsv"])
        if marks:
            marks[1].record(stream)
        if d["nv"]:
            S.pillar_topk(st["logits"], d["lse_v"], st["lstride"], d["seq_v"], self.ctxs[i], d["nv"], w.batch,
                          self.max_ctx, hq, hkv, k, self.s, st["sel"], self.sel_stride, st["cnt"], st["sl"], st["wst"])
        if marks:
            marks[2].record(stream)
        if d["nd"]:
            S.sparse_draft_attn(self.kv, d["qd"], d["seq_d"], self.ctxs[i], st["sel"], self.sel_stride, st["cnt"],
                                st["sl"], d["nd"], self.max_ctx, hq, w.sm_scale, d["out_d"], d["lse_d"], st["wsd"])
        if marks:
            marks[3].record(stream)

    def bytes_and_queries(self, steps):
        w = self.w
        sc = self.cnt.cpu().numpy()
        q = b = 0
        for t in range(steps):
            vb, isv, ctx, step = self.cycles[t % self.kp1]
            q += int(np.where(isv, self.kp1, 1).sum())
            b += algorithmic_bytes(w.verify_lens, isv, step, sc, w.k, self.s, w.num_q_heads, w.num_kv_heads)
        return b, q

    def time_steps(self, steps, fn):
        """Run fn(t) for t in [0, steps) between events on the current stream:
        (total ms, per-step ms list)."""
        torch = self.torch
        stream = torch.cuda.current_stream()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record(stream)
        for t in range(steps):
            ev[t][0].record(stream)
            fn(t)
            ev[t][1].record(stream)
        t1.record(stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1), [a.elapsed_time(b) for a, b in ev]


class LayerHarness(Harness):
    """Unified launches of decode steps through `layers` attention layers.
    Every layer has KV pools of its own (copies of the generated pools at
    their own addresses, so no layer reads what another left in the
    caches), its own query rows, outputs and selection state; the
    workspace is shared, as a model's layers run one after another.  Launch
    t runs layer t mod layers on verify bucket (t div layers) mod k+1:
    every layer of one decode step, then the next step."""

    def __init__(self, S, w, s, layers, dev="cuda"):
        super().__init__(S, w, s, dev)
        torch = self.torch
        self.layers = layers
        self.per = [dict(kv=self.kv, qs=self.qs, outs=self.outs, lses=self.lses, sel=self.sel, cnt=self.cnt,
                         sl=self.sl)]
        for _ in range(layers - 1):
            self.per.append(dict(
                kv=S.PagedKV(w.k_pages.clone(), w.v_pages.clone(), w.block_table),
                qs=[q.clone() for q in self.qs], outs=[torch.empty_like(o) for o in self.outs],
                lses=[torch.empty_like(x) for x in self.lses], sel=torch.zeros_like(self.sel),
                cnt=torch.zeros_like(self.cnt), sl=self.sl.clone()))

    def launch(self, t):
        w, P, i = self.w, self.per[t % self.layers], (t // self.layers) % self.kp1
        self.S.unified_attn(P["kv"], P["qs"][i], self.ctxs[i], self.bk, self.cycles[i][0], w.batch,
                            self.max_verify, self.max_ctx, w.num_q_heads, w.k, self.s, w.sm_scale, P["sel"],
                            self.sel_stride, P["cnt"], P["sl"], P["outs"][i], P["lses"][i], self.ws)

    def setup_cycle(self):
        for t in range(self.kp1 * self.layers):   # every request verifies once in every layer
            self.launch(t)
        self.torch.cuda.synchronize()
        flags = self.S.read_device_error(self.ws)
        if flags:
            raise RuntimeError(f"device error flags 0x{flags:x} in the set-up cycle")

    def bytes_and_queries(self, steps):
        w = self.w
        counts = [P["cnt"].cpu().numpy() for P in self.per]
        q = b = 0
        for t in range(steps):
            vb, isv, ctx, step = self.cycles[(t // self.layers) % self.kp1]
            q += int(np.where(isv, self.kp1, 1).sum())
            b += algorithmic_bytes(w.verify_lens, isv, step, counts[t % self.layers], w.k, self.s,
                                   w.num_q_heads, w.num_kv_heads)
        return b, q


def torch_empty_like(t):
    import torch
    return torch.empty_like(t)


def copy_bandwidth(torch, dev, mib=2048, reps=5):
    """Device-to-device copy of mib MiB, best of reps: GB/s of read + write bytes."""
    n = mib << 18
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    best = 0.0
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        best = max(best, 2 * n * 4 / (a.elapsed_time(b) / 1e3) / 1e9)
    del src, dst
    torch.cuda.empty_cache()
    return best


def base_record(metric, value, unit, steps, warmup, ms_per_step, config):
    return {"metric": metric, "value": value, "unit": unit, "n_gpus": 1, "steps": steps, "warmup": warmup,
            "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "bf16", "data": "synthetic", "config": config}


def workload_config(spec, w, s, seed, extra=None):
    c = {"workload": spec["name"], "batch": w.batch, "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads,
         "head_dim": 128, "page_size": 16, "k": w.k, "s": s, "mean_verify_ctx": float(w.verify_lens.mean()),
         "max_ctx": int(w.caps.max()), "seed": seed}
    c.update(extra or {})
    return c


# ------------------------------------------------------------------ modes
def calibration_copy(torch, mib):
    """One device copy of mib MiB: a known-size reference for HBM traffic counters."""
    n = mib << 18   # float32 elements
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    log(f"calibration copy: {mib} MiB read + {mib} MiB written")
    del src, dst
    torch.cuda.empty_cache()


def run_unified(args, torch, S, spec, w):
    h = Harness(S, w, w.s)
    h.setup_cycle()
    for t in range(args.warmup):
        h.launch(t)
    total_ms, kern_ms = h.time_steps(args.steps, h.launch)
    flags = S.read_device_error(h.ws)
    if flags:
        raise RuntimeError(f"device error flags 0x{flags:x} in the timed region")
    alg_bytes, queries = h.bytes_and_queries(args.steps)
    value = queries / (total_ms / 1e3)
    mean_kern_s = float(np.mean(kern_ms)) / 1e3
    bytes_per_launch = alg_bytes / args.steps
    achieved = bytes_per_launch / mean_kern_s / 1e9
    achieved_step = alg_bytes / (total_ms / 1e3) / 1e9
    copy_gbps = copy_bandwidth(torch, "cuda") if not args.no_copy_ref else None

    traffic = None
    prof = os.path.join(ROOT, "profiles", "unified_kernel_qwen3-8b_B128_traffic.json")
    if os.path.exists(prof):
        with open(prof) as f:
            tr = json.load(f)
        if tr.get("kernel_source_digest") == kernel_source_digest():
            traffic = tr.get("hbm_bytes_per_launch")

    cpu = None
    if not args.no_cpu:
        from sspec_workload import to_numpy_bf16
        kp, vp, bt = to_numpy_bf16(w.k_pages), to_numpy_bf16(w.v_pages), w.block_table.cpu().numpy()
        cpu = cpu_baseline(w, kp, vp, bt, h.cycles[0], args.cpu_budget)

    rot, part = divmod(args.steps, h.kp1)
    metric = METRIC if args.config == 2 else f"unified attn queries/s + achieved HBM GB/s (% of peak), {spec['name']}"
    rec = base_record(metric, value, "queries/s", args.steps, args.warmup, total_ms / args.steps,
                      workload_config(spec, w, w.s, args.seed, {
                          "queries_per_step": queries / args.steps,
                          # value and bytes are those of exactly the steps timed: a partial
                          # rotation is counted with its own verify bucket's sizes
                          "full_rotations": rot, "partial_rotation_steps": part}))
    rec.update({
        "hbm_gbps": achieved,
        "hbm_frac_of_peak": achieved / PEAK_HBM_GBS,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": traffic,
                     "kernel": "unified_kernel", "alg_bytes_per_launch": bytes_per_launch,
                     "mean_launch_us": mean_kern_s * 1e6,
                     # the same bytes over the whole timed region (launch gaps included)
                     "achieved_from_step_time": achieved_step,
                     "frac_from_step_time": achieved_step / PEAK_HBM_GBS,
                     # a device-to-device copy measured in this run: the bandwidth a
                     # plain streaming kernel reaches on this GPU
                     "copy_gbps": copy_gbps,
                     "frac_of_copy": (achieved / copy_gbps) if copy_gbps else None},
        "cpu_baseline": cpu,
    })
    print(json.dumps(rec), flush=True)


def run_layers(args, torch, S, spec, w):
    """Unified launches cycling over the KV caches of several attention
    layers (as many as fit in device memory, up to --kv-layers), so that the
    footprint is a model's rather than one layer's.  A step is one decode
    step through every layer (`layers` launches); the value counts the
    queries of every launch, like the one-layer rate."""
    per_layer = 2 * w.k_pages.numel() * w.k_pages.element_size()
    free, _ = torch.cuda.mem_get_info()
    fit = 1 + max(0, int((free - (8 << 30)) // per_layer))
    layers = max(1, min(args.kv_layers, fit))
    if layers < args.kv_layers:
        log(f"{args.kv_layers} layers of {per_layer / 1e9:.1f} GB pools do not fit in {free / 1e9:.0f} GB free: "
            f"{layers} layers")
    h = LayerHarness(S, w, w.s, layers)
    h.setup_cycle()
    log(f"{layers} layers set up: {layers * per_layer / 1e9:.1f} GB of KV pools")
    for t in range(args.warmup * layers):
        h.launch(t)
    n = args.steps * layers
    total_ms, kern_ms = h.time_steps(n, h.launch)
    flags = S.read_device_error(h.ws)
    if flags:
        raise RuntimeError(f"device error flags 0x{flags:x} in the timed region")
    alg_bytes, queries = h.bytes_and_queries(n)
    mean_kern_s = float(np.mean(kern_ms)) / 1e3
    achieved = alg_bytes / n / mean_kern_s / 1e9
    rec = base_record(f"unified attn queries/s per attention layer, {layers} layers' KV caches cycled",
                      queries / (total_ms / 1e3), "queries/s", args.steps, args.warmup, total_ms / args.steps,
                      workload_config(spec, w, w.s, args.seed, {
                          "kv_layers": layers, "kv_layers_requested": args.kv_layers,
                          "kv_pool_bytes_per_layer": per_layer, "launches_per_step": layers,
                          "queries_per_launch": queries / n}))
    rec.update({
        "us_per_launch": total_ms / n * 1e3,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": None, "kernel": "unified_kernel",
                     "alg_bytes_per_launch": alg_bytes / n, "mean_launch_us": mean_kern_s * 1e6},
    })
    print(json.dumps(rec), flush=True)


def run_separate(args, torch, S, spec, w, s=None, extra=None, h=None, check_full=False):
    """Unified vs the three separate launches on the same steps; returns the record."""
    s = w.s if s is None else s
    h = h or Harness(S, w, s)
    h.setup_cycle()
    for t in range(args.warmup):
        h.launch(t)
        h.launch_separate(t)
    torch.cuda.synchronize()
    steps = args.steps
    tot_u, kern_u = h.time_steps(steps, h.launch)
    marks = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    tot_s, _ = h.time_steps(steps, lambda t: h.launch_separate(t, marks[t]))
    parts = np.array([[m[0].elapsed_time(m[1]), m[1].elapsed_time(m[2]), m[2].elapsed_time(m[3])] for m in marks])
    for ws in (h.ws, h._sep["wsv"], h._sep["wst"], h._sep["wsd"]):
        flags = S.read_device_error(ws)
        if flags:
            raise RuntimeError(f"device error flags 0x{flags:x}")
    alg_bytes, queries = h.bytes_and_queries(steps)
    u_us, s_us = tot_u / steps * 1e3, tot_s / steps * 1e3
    achieved = alg_bytes / steps / (float(np.mean(kern_u)) / 1e3) / 1e9
    rec = base_record("unified vs separate launches: queries/s", queries / (tot_u / 1e3), "queries/s", steps,
                      args.warmup, tot_u / steps, workload_config(spec, w, s, args.seed, extra))
    rec.update({
        "unified_us_per_step": u_us, "separate_us_per_step": s_us, "speedup_unified_vs_separate": s_us / u_us,
        "separate_parts_us": {"verify": float(parts[:, 0].mean() * 1e3), "pillar_topk": float(parts[:, 1].mean() * 1e3),
                              "draft": float(parts[:, 2].mean() * 1e3)},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": None, "kernel": "unified_kernel",
                     "alg_bytes_per_launch": alg_bytes / steps, "mean_launch_us": float(np.mean(kern_u)) * 1e3},
    })
    if check_full:
        rec["s1_full_attention_max_abs_err"] = full_attention_check(torch, h)
    return rec


def run_naive(args, torch, S, spec, w):
    """Fused launch vs the naive-batching launch (every item in the verify's
    tile shape) vs the three separate launches, on the same steps."""
    h = Harness(S, w, w.s)
    rec = run_separate(args, torch, S, spec, w, h=h)
    for t in range(h.kp1):   # the naive path's own selection state, then warm-up
        h.launch_naive(t)
    for t in range(args.warmup):
        h.launch_naive(t)
    torch.cuda.synchronize()
    tot_n, kern_n = h.time_steps(args.steps, h.launch_naive)
    flags = S.read_device_error(h._naive[0])
    if flags:
        raise RuntimeError(f"device error flags 0x{flags:x} (naive)")
    n_us = tot_n / args.steps * 1e3
    rec["metric"] = "fused vs naive-batching vs separate launches: queries/s"
    rec["naive_us_per_step"] = n_us
    rec["speedup_fused_vs_naive"] = n_us / rec["unified_us_per_step"]
    # the naive launch moves the same algorithmic bytes
    rec["naive_roofline_frac"] = rec["roofline"]["alg_bytes_per_launch"] / (float(np.mean(kern_n)) / 1e3) / 1e9 \
        / PEAK_HBM_GBS
    return rec


def run_offload(args, torch, S, spec, w):
    """Unified launches of the benchmark rotation with the KV offload engine
    moving a cold pool's pages to host memory and back on a side stream,
    at several offload rates (pages per launch), against no offload."""
    h = Harness(S, w, w.s)
    h.setup_cycle()
    hkv = w.num_kv_heads
    pb = S.offload_page_bytes(hkv)
    chunk, slots, job_pages, n_cold = 32, 4, 64, 2048
    g = torch.Generator(device="cuda").manual_seed(1)
    cold_k = torch.randn(n_cold, hkv, 16, 128, generator=g, device="cuda").to(torch.bfloat16)
    cold_v = torch.randn(n_cold, hkv, 16, 128, generator=g, device="cuda").to(torch.bfloat16)
    cold = S.PagedKV(cold_k, cold_v, torch.zeros(1, 1, dtype=torch.int32, device="cuda"))
    staging = torch.empty(slots * chunk * pb, dtype=torch.uint8, device="cuda")
    host = torch.empty(S.offload_host_bytes(hkv, chunk, slots, n_cold), dtype=torch.uint8, pin_memory=True)
    side = torch.cuda.Stream()
    njobs = n_cold // job_pages
    stream = torch.cuda.current_stream()
    recs = []
    for pages_per_step in [0] + [int(x) for x in args.offload_rates.split(",")]:
        eng = S.Offload(cold, chunk, slots, staging=staging, host=host, side_stream=side)
        # cold "requests" cycle: on the device -> evicted (host copy) -> restored;
        # a few jobs are kept queued, and chunks are issued as the byte budget of
        # the rate allows
        state = {"on_dev": list(range(njobs)), "evicted": [], "moved": 0, "budget": 0.0, "ev": []}

        def feed():
            jobs, _, _ = eng.pending()
            while jobs < 4:
                if len(state["evicted"]) < njobs // 2 and state["on_dev"]:
                    j = state["on_dev"].pop(0)
                    eng.evict(j, list(range(j * job_pages, (j + 1) * job_pages)))
                    state["evicted"].append(j)
                elif state["evicted"]:
                    j = state["evicted"].pop(0)
                    eng.restore(j, list(range(j * job_pages, (j + 1) * job_pages)))
                else:
                    break
                jobs += 1

        def step(t):
            h.launch(t)
            # pace the host like a serving loop: at most two launches in flight
            ev = torch.cuda.Event()
            ev.record(stream)
            state["ev"].append(ev)
            if len(state["ev"]) > 2:
                state["ev"].pop(0).synchronize()
            if pages_per_step:
                feed()
                state["budget"] += pages_per_step / chunk
                n = int(state["budget"])
                if n:
                    eng.pump(n)
                    state["budget"] -= n
                for req, kind in eng.poll():
                    state["moved"] += job_pages
                    if kind == S.OFFLOAD_RESTORE:
                        state["on_dev"].append(req)

        for t in range(args.warmup):
            step(t)
        torch.cuda.synchronize()
        state["moved"] = 0
        t0 = time.perf_counter()
        total_ms, kern_ms = h.time_steps(args.steps, step)
        wall = time.perf_counter() - t0
        moved = state["moved"] * pb
        eng.close()
        side.synchronize()
        recs.append({"pages_per_step": pages_per_step, "ms_per_step": total_ms / args.steps,
                     "launch_us": float(np.mean(kern_ms)) * 1e3, "offload_gbps": moved / wall / 1e9,
                     "offload_mb_per_step": moved / args.steps / 1e6})
        log(f"offload {pages_per_step} pages/step: {recs[-1]}")
    base = recs[0]["ms_per_step"]
    for r in recs:
        r["overhead_pct"] = (r["ms_per_step"] / base - 1.0) * 100.0
    alg_bytes, queries = h.bytes_and_queries(args.steps)
    rec = base_record("unified attn step time with concurrent KV offload: queries/s", queries / (base / 1e3 * args.steps),
                      "queries/s", args.steps, args.warmup, base,
                      workload_config(spec, w, w.s, args.seed, {"page_bytes": pb, "chunk_pages": chunk,
                                                                 "job_pages": job_pages}))
    rec["offload"] = recs
    return rec


def run_loop(args, torch, S, spec, w):
    """A decode loop driven by the native scheduler: per iteration the batch
    is formed on the host, then `layers` times (KV append by slot + unified
    launch by slot), then the acceptance stub and the copy of its result to
    the host.  Synchronous mode waits for each iteration's result before
    forming the next; delayed verification reads it one iteration late."""
    import math as _m
    B, hq, hkv, k = w.batch, w.num_q_heads, w.num_kv_heads, w.k
    L = args.layers
    iters = args.loop_iters
    kv = S.PagedKV(w.k_pages, w.v_pages, w.block_table)
    max_ctx = int(w.caps.max())
    sel_stride = _m.ceil(w.s * max_ctx)
    rows_max = B * (k + 1)
    g = torch.Generator(device="cuda").manual_seed(2)
    qbuf = torch.randn(rows_max, hq, 128, generator=g, device="cuda").to(torch.bfloat16)
    knew = torch.randn(rows_max, hkv, 128, generator=g, device="cuda").to(torch.bfloat16)
    vnew = torch.randn(rows_max, hkv, 128, generator=g, device="cuda").to(torch.bfloat16)
    out = torch.empty_like(qbuf)
    lse = torch.empty(rows_max, hq, dtype=torch.float32, device="cuda")
    res = {}
    for delayed in (False, True):
        # the pools are only read (positions below each request's original
        # context) and overwritten by the appends: both modes see valid data
        sched = S.Scheduler(k, B, delayed=delayed)
        for r in range(B):
            sched.admit(r, int(w.verify_lens[r]) - iters - 2, 1 << 30)
        mv = int(np.bincount(w.bucket_ids, minlength=k + 1).max()) + 1
        ws = S.workspace(S.unified_workspace_size(B, mv, max_ctx, hq, hkv, k))
        sel = torch.zeros(B, hkv, sel_stride, dtype=torch.int32, device="cuda")
        cnt = torch.zeros(B, dtype=torch.int32, device="cuda")
        acc_d = torch.zeros(B, dtype=torch.int32, device="cuda")
        pin = [[torch.zeros(B, dtype=torch.int32).pin_memory() for _ in range(5)] for _ in range(2)]
        dev = [[torch.zeros(B, dtype=torch.int32, device="cuda") for _ in range(5)] for _ in range(2)]
        acc_h = [torch.zeros(B, dtype=torch.int32).pin_memory() for _ in range(2)]
        evs = [torch.cuda.Event() for _ in range(2)]
        host_s = 0.0
        prev = None
        wall0 = None
        def committed():
            return sum(sched.query(x)[2] for x in range(B))

        for t in range(iters):
            if t == args.warmup:
                torch.cuda.synchronize()
                wall0 = time.perf_counter()
                host_s = 0.0
                tok0 = committed()
            b = t % 2
            h0 = time.perf_counter()
            req, seq, bk, ctx, sl = pin[b]
            it, vb, n, nv = sched.next(req, seq, bk, ctx, sl)
            host_s += time.perf_counter() - h0
            for src, dst in zip(pin[b], dev[b]):
                dst.copy_(src, non_blocking=True)
            req_d, seq_d, bk_d, ctx_d, sl_d = dev[b]
            rows = n + k * nv
            for _ in range(L):
                S.kv_append_slots(kv, knew[:rows], vnew[:rows], seq_d, ctx_d, bk_d, vb, n, k)
                S.unified_attn_slots(kv, qbuf[:rows], seq_d, ctx_d, bk_d, vb, n, mv, max_ctx, hq, k, w.s, w.sm_scale,
                                     sel, sel_stride, cnt, sl_d, out[:rows], lse[:rows], ws)
            if nv:
                S.accept_stub(req_d, seq_d, bk_d, vb, n, k, it, 0.742, 5, B, acc_d)
            acc_h[b].copy_(acc_d, non_blocking=True)
            evs[b].record()
            cur = (it, b)
            wait = (prev if delayed else cur)
            if delayed:
                prev = cur
            if wait is not None:
                evs[wait[1]].synchronize()
                h0 = time.perf_counter()
                sched.resolve(wait[0], acc_h[wait[1]].numpy())
                host_s += time.perf_counter() - h0
            if args.host_work_ms > 0:
                # stand-in for the rest of the host's per-iteration work
                # (sampling, detokenisation, request bookkeeping): a busy wait
                end = time.perf_counter() + args.host_work_ms / 1e3
                while time.perf_counter() < end:
                    pass
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        flags = S.read_device_error(ws)
        if flags:
            raise RuntimeError(f"device error flags 0x{flags:x} (loop)")
        n_it = iters - args.warmup
        # tokens committed by the verifies resolved in the timed iterations
        toks = committed() - tok0
        res["delayed" if delayed else "sync"] = {"ms_per_iteration": wall / n_it * 1e3,
                                                 "host_sched_us_per_iteration": host_s / n_it * 1e6,
                                                 "committed_tokens_per_s": toks / wall}
        log(f"loop delayed={delayed}: {res['delayed' if delayed else 'sync']}")
    rec = base_record("decode iterations/s (scheduler-driven loop, delayed verification)",
                      1e3 / res["delayed"]["ms_per_iteration"], "iterations/s", iters - args.warmup, args.warmup,
                      res["delayed"]["ms_per_iteration"],
                      workload_config(spec, w, w.s, args.seed, {"layers": L, "acceptance_rate": 0.742,
                                                                 "host_work_ms": args.host_work_ms}))
    rec.update(res)
    rec["speedup_delayed_vs_sync"] = res["sync"]["ms_per_iteration"] / res["delayed"]["ms_per_iteration"]
    rec["token_speedup_delayed_vs_sync"] = (res["delayed"]["committed_tokens_per_s"]
                                            / max(res["sync"]["committed_tokens_per_s"], 1e-9))
    return rec


def full_attention_check(torch, h):
    """At s = 1 a draft attends to its whole context: compare one sampled
    draft output of the last unified launch with plain full attention in
    torch (fp32 over the bf16 inputs, gathered through the block table)."""
    w = h.w
    t = h.kp1 - 1   # the last step of the timed rotation: its outputs are in outs[t]
    vb, isv, ctx, step = h.cycles[t]
    did = np.nonzero(~isv)[0]
    r = int(did[len(did) // 2])
    off = int(np.concatenate([[0], np.cumsum(np.where(isv, h.kp1, 1))])[r])
    L = int(ctx[r])
    pages = w.block_table[r, : -(-L // 16)].long()
    kc = w.k_pages[pages].float().permute(1, 0, 2, 3).reshape(w.num_kv_heads, -1, 128)[:, :L]
    vc = w.v_pages[pages].float().permute(1, 0, 2, 3).reshape(w.num_kv_heads, -1, 128)[:, :L]
    q = h.qs[t][off].float()                                   # [hq][128]
    G = w.num_q_heads // w.num_kv_heads
    kx = kc.repeat_interleave(G, dim=0)
    vx = vc.repeat_interleave(G, dim=0)
    p = torch.softmax((kx @ q[:, :, None]).squeeze(-1) * float(np.float32(w.sm_scale)), dim=-1)
    o = (p[:, None, :] @ vx).squeeze(1)
    return float((h.outs[t][off].float() - o).abs().max())


def run_kv_append(args, torch, S, spec, w):
    """sspec_kv_append of every step's rows of the rotation."""
    from sspec_workload import cycle_state
    k, hkv, B = w.k, w.num_kv_heads, w.batch
    kp1 = k + 1
    kv = S.PagedKV(w.k_pages, w.v_pages, w.block_table)
    bk = torch.from_numpy(w.bucket_ids).to("cuda")
    cyc = [cycle_state(w, t) for t in range(kp1)]
    ctxs = [torch.from_numpy(c[2].astype(np.int32)).to("cuda") for c in cyc]
    rows = [int(np.where(c[1], kp1, 1).sum()) for c in cyc]
    g = torch.Generator(device="cuda").manual_seed(1)
    news = [(torch.randn(n, hkv, 128, generator=g, device="cuda").to(torch.bfloat16),
             torch.randn(n, hkv, 128, generator=g, device="cuda").to(torch.bfloat16)) for n in rows]
    err = torch.zeros(1, dtype=torch.int32, device="cuda")

    def launch(t):
        i = t % kp1
        S.kv_append(kv, news[i][0], news[i][1], ctxs[i], bk, cyc[i][0], B, k, err=err)

    for t in range(args.warmup + kp1):
        launch(t)
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for t in range(args.steps):
        ev[t][0].record(stream)
        launch(t)
        ev[t][1].record(stream)
    t1.record(stream)
    torch.cuda.synchronize()
    if int(err.item()):
        raise RuntimeError(f"kv_append error bits 0x{int(err.item()):x}")
    total_ms = t0.elapsed_time(t1)
    kern = float(np.mean([a.elapsed_time(b) for a, b in ev])) / 1e3
    nrows = sum(rows[t % kp1] for t in range(args.steps))
    # per row and KV head: 256 B of K and 256 B of V read from the new rows and
    # written to the pages; plus ctx_lens and bucket ids (4 + 4 B per request)
    alg = (nrows * hkv * 2 * 256 * 2 + args.steps * B * 8) / args.steps
    rec = base_record("kv append rows/s (one unified iteration's K/V into the paged cache)",
                      nrows / (total_ms / 1e3), "rows/s", args.steps, args.warmup, total_ms / args.steps,
                      workload_config(spec, w, w.s, args.seed, {"rows_per_step": nrows / args.steps}))
    # the same event pair around a kernel that does (almost) nothing: the
    # fixed cost any launch of this size pays on this GPU
    tiny = torch.zeros(64, dtype=torch.int32, device="cuda")
    fl = []
    for _ in range(50):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        tiny.zero_()
        b.record(stream)
        fl.append((a, b))
    torch.cuda.synchronize()
    floor_us = float(np.median([a.elapsed_time(b) for a, b in fl])) * 1e3
    rec["roofline"] = {"bound": "hbm", "achieved": alg / kern / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                       "frac": alg / kern / 1e9 / PEAK_HBM_GBS, "traffic": None, "kernel": "kv_append_kernel",
                       "alg_bytes_per_launch": alg, "mean_launch_us": kern * 1e6,
                       "ideal_us_at_peak": alg / (PEAK_HBM_GBS * 1e9) * 1e6,
                       "empty_kernel_us": floor_us}
    print(json.dumps(rec), flush=True)


def run_sweep(args, torch, S):
    from sspec_workload import make_workload, workload_spec
    Ls = [int(x) for x in args.sweep_L.split(",")]
    ks = [int(x) for x in args.sweep_k.split(",")]
    ss = [float(x) for x in args.sweep_s.split(",")]
    for L in Ls:
        for k in ks:
            spec = workload_spec(4, lengths=("fixed", L), k=k)
            t0 = time.time()
            w = make_workload(spec, seed=4, device="cuda")
            torch.cuda.synchronize()
            log(f"sweep workload L={L} k={k} generated in {time.time() - t0:.1f}s")
            for s in ss:
                rec = run_separate(args, torch, S, spec, w, s=s, extra={"L": L, "sweep": True},
                                   check_full=(s == 1.0))
                print(json.dumps(rec), flush=True)
                torch.cuda.empty_cache()
            del w
            torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=90)
    ap.add_argument("--warmup", type=int, default=9)
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--seed", type=int, default=2)
    ap.add_argument("--bench", choices=["unified", "separate", "naive", "kv_append", "sweep", "offload", "loop",
                                        "layers"],
                    default="unified")
    ap.add_argument("--offload-rates", default="8,32,128",
                    help="offload mode: pages moved per launch (8 ~ 18 MB per 36-layer decode step)")
    ap.add_argument("--layers", type=int, default=36, help="loop mode: attention layers per iteration")
    ap.add_argument("--loop-iters", type=int, default=24, help="loop mode: iterations (warm-up included)")
    ap.add_argument("--host-work-ms", type=float, default=0.0,
                    help="loop mode: emulated host work per iteration besides the scheduler (busy wait)")
    ap.add_argument("--kv-layers", type=int, default=36,
                    help="layers mode: attention layers whose KV caches the launches cycle over (as many as fit)")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-copy-ref", action="store_true", help="skip the device-copy reference bandwidth")
    ap.add_argument("--sweep-L", default="65536,131072")
    ap.add_argument("--sweep-k", default="4,8,16")
    ap.add_argument("--sweep-s", default="0.01,0.05,0.1,1.0")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="also run one device copy of this many MiB (a known-size reference "
                         "for the HBM traffic counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import torch
    from sparse_self_speculative_amd import sspec as S
    from sspec_workload import make_workload, workload_spec

    if args.calib_copy_mb:
        calibration_copy(torch, args.calib_copy_mb)
    if args.bench == "sweep":
        run_sweep(args, torch, S)
        return
    spec = workload_spec(args.config)
    t0 = time.time()
    w = make_workload(spec, seed=args.seed, device="cuda")
    torch.cuda.synchronize()
    log(f"workload {spec['name']}: B={w.batch} mean L={w.verify_lens.mean():.0f} "
        f"pages={w.num_pages} generated in {time.time() - t0:.1f}s")
    if args.steps % (w.k + 1):
        log(f"note: {args.steps} steps are not whole rotations of {w.k + 1}; the figures are those of "
            f"exactly the steps timed")
    if args.bench == "unified":
        run_unified(args, torch, S, spec, w)
    elif args.bench == "separate":
        print(json.dumps(run_separate(args, torch, S, spec, w)), flush=True)
    elif args.bench == "naive":
        print(json.dumps(run_naive(args, torch, S, spec, w)), flush=True)
    elif args.bench == "offload":
        print(json.dumps(run_offload(args, torch, S, spec, w)), flush=True)
    elif args.bench == "loop":
        print(json.dumps(run_loop(args, torch, S, spec, w)), flush=True)
    elif args.bench == "layers":
        run_layers(args, torch, S, spec, w)
    else:
        run_kv_append(args, torch, S, spec, w)


if __name__ == "__main__":
    main()

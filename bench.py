"""Benchmark of the unified SparseSpec attention launch on one MI355X.

Workload (default): Qwen3-8B attention shape (32 query / 8 KV heads,
head_dim 128, bf16), batch 128, verify-time context lengths lognormal with
mean 12000 and sd 7600 clipped to [1024, 32768], k = 8, s = 0.05, page 16,
requests spread over k+1 buckets by least-loaded assignment.  One step is
one unified launch (one attention layer): the requests of one bucket verify
(k+1 queries, full attention, logit+LSE dump, PillarAttn Top-K) and all the
others run one sparse draft step.  Timed steps rotate the verify bucket, so
every full cycle of k+1 steps verifies each request once.

Prints ONE JSON line: queries/s (one query = one query token of one request
across all heads), the achieved algorithmic HBM bandwidth of the unified
kernel against the 8 TB/s peak, and the CPU oracle timed on a bounded
sample on this host.
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=90)
    ap.add_argument("--warmup", type=int, default=9)
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--seed", type=int, default=2)
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--no-cpu", action="store_true")
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
    from sspec_workload import cycle_state, make_workload, pack_rows, to_numpy_bf16, workload_spec

    dev = "cuda"
    spec = workload_spec(args.config)
    t0 = time.time()
    w = make_workload(spec, seed=args.seed, device=dev)
    torch.cuda.synchronize()
    log(f"workload {spec['name']}: B={w.batch} mean L={w.verify_lens.mean():.0f} "
        f"pages={w.num_pages} generated in {time.time() - t0:.1f}s")
    B, hq, hkv, k, s = w.batch, w.num_q_heads, w.num_kv_heads, w.k, w.s
    kp1 = k + 1
    max_ctx = int(w.caps.max())
    sel_stride = math.ceil(s * max_ctx)
    max_verify = int(np.bincount(w.bucket_ids, minlength=kp1).max())
    kv = S.PagedKV(w.k_pages, w.v_pages, w.block_table)
    ws = S.workspace(S.unified_workspace_size(B, max_verify, max_ctx, hq, hkv, k), dev)
    sel_idx = torch.zeros(B, hkv, sel_stride, dtype=torch.int32, device=dev)
    sel_count = torch.zeros(B, dtype=torch.int32, device=dev)
    sel_len = torch.from_numpy(w.verify_lens.astype(np.int32)).to(dev)
    buckets = torch.from_numpy(w.bucket_ids).to(dev)
    cycles = [cycle_state(w, t) for t in range(kp1)]
    qs = [pack_rows(w, c[1], c[3], dev) for c in cycles]
    ctxs = [torch.from_numpy(c[2].astype(np.int32)).to(dev) for c in cycles]
    outs = [torch.empty_like(q) for q in qs]
    lses = [torch.empty(q.shape[0], hq, dtype=torch.float32, device=dev) for q in qs]

    def launch(t):
        i = t % kp1
        S.unified_attn(kv, qs[i], ctxs[i], buckets, cycles[i][0], B, max_verify, max_ctx, hq, k, s,
                       w.sm_scale, sel_idx, sel_stride, sel_count, sel_len, outs[i], lses[i], ws)

    if args.calib_copy_mb:
        n = args.calib_copy_mb << 18   # float32 elements
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy: {args.calib_copy_mb} MiB read + {args.calib_copy_mb} MiB written")
        del src, dst

    # set-up cycle: every request verifies once, so every draft holds a selection
    for t in range(kp1):
        launch(t)
    for t in range(args.warmup):
        launch(t)
    torch.cuda.synchronize()
    flags = S.read_device_error(ws)
    if flags:
        raise RuntimeError(f"device error flags 0x{flags:x} after warm-up")

    sc = sel_count.cpu().numpy()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for t in range(args.steps):
        ev[t][0].record(stream)
        launch(t)
        ev[t][1].record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    kern_ms = [a.elapsed_time(b) for a, b in ev]
    flags = S.read_device_error(ws)
    if flags:
        raise RuntimeError(f"device error flags 0x{flags:x} in the timed region")

    queries = 0
    alg_bytes = 0
    for t in range(args.steps):
        vb, isv, ctx, step = cycles[t % kp1]
        queries += int(np.where(isv, kp1, 1).sum())
        alg_bytes += algorithmic_bytes(w.verify_lens, isv, step, sc, k, s, hq, hkv)
    value = queries / (total_ms / 1e3)
    mean_kern_s = float(np.mean(kern_ms)) / 1e3
    bytes_per_launch = alg_bytes / args.steps
    achieved = bytes_per_launch / mean_kern_s / 1e9

    traffic = None
    prof = os.path.join(ROOT, "profiles", "unified_kernel_qwen3-8b_B128_traffic.json")
    if os.path.exists(prof):
        with open(prof) as f:
            tr = json.load(f)
        if tr.get("kernel_source_digest") == kernel_source_digest():
            traffic = tr.get("hbm_bytes_per_launch")

    cpu = None
    if not args.no_cpu:
        kp, vp, bt = to_numpy_bf16(w.k_pages), to_numpy_bf16(w.v_pages), w.block_table.cpu().numpy()
        cpu = cpu_baseline(w, kp, vp, bt, cycles[0], args.cpu_budget)

    rec = {
        "metric": "unified attn queries/s + achieved HBM GB/s (% of peak), Qwen3-8B shape, B=128",
        "value": value,
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": total_ms / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": spec["name"], "batch": B, "num_q_heads": hq, "num_kv_heads": hkv,
                   "head_dim": 128, "page_size": 16, "k": k, "s": s,
                   "mean_verify_ctx": float(w.verify_lens.mean()), "max_ctx": max_ctx,
                   "queries_per_step": queries / args.steps, "seed": args.seed},
        "hbm_gbps": achieved,
        "hbm_frac_of_peak": achieved / PEAK_HBM_GBS,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": traffic,
                     "kernel": "unified_kernel", "alg_bytes_per_launch": bytes_per_launch,
                     "mean_launch_us": mean_kern_s * 1e6},
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()

"""Seeded synthetic workloads shaped like the SparseSpec evaluation.

Source pages: "Accelerating Large-Scale Reasoning Model Inference with Sparse
Self-Speculative Decoding" (MLSys 2026 talk notes).  The models used there
are Qwen3-1.7B/8B/14B (section "Experimental setup", paper Table 2); the
output-length statistics that shape the context-length draws are in section
"Problem setting" (paper Table 1: Qwen3-14B on AIME has mean 13,542 and
standard deviation 7,626 tokens; Qwen3-8B averages 12K).  The request
buckets follow section "Unified batch scheduler" (paper §4.2, Fig. 8): k+1
buckets, new requests go to the least-loaded one.  None of the datasets is
used; only their length statistics are.

What is generated (all from one integer seed):
  * K, V ~ N(0, 1) in float32, rounded to bfloat16 (round to nearest even,
    which is what torch's float32 -> bfloat16 conversion does).
  * "Pillar" tokens: for every (request, KV head) a random unit direction u
    and round(pillar_frac * L) distinct positions in [0, L).  Those key rows
    get + pillar_k_shift * u, and every query of that KV head's group gets
    + q_shift * u, so the pillars carry a logit boost of about
    pillar_k_shift * q_shift / sqrt(d) (3 with the defaults).
  * Physical pages are a seeded permutation of the pool, so block tables are
    not contiguous.
  * Per request a bank of 2k+1 query rows: rows 0..k are the verify queries
    (positions L-k-1 .. L-1) and row k+j is the query of draft step j
    (position L+j-1), j = 1..k.  Pages hold L+k tokens so every draft step
    has its own key/value row written.

No attention, scoring or selection arithmetic lives here.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np
import torch

# (query heads, KV heads) of the attention layers of the evaluated models
# (head_dim 128 for all three).
ATTN_SHAPES: Dict[str, tuple] = {
    "qwen3-1.7b": (16, 8),
    "qwen3-8b": (32, 8),
    "qwen3-14b": (40, 8),
}


def workload_spec(index: int, **overrides) -> dict:
    """The five synthetic workloads, by index.

    0: one request, L = 2048, 16/8 heads, k = 8, s = 0.05.
    1: Qwen3-1.7B shape, batch 64, L uniform on [4096, 16384].
    2: Qwen3-8B shape, batch 128, L lognormal (mean 12000, sd 7600) clipped
       to [1024, 32768].
    3: Qwen3-14B shape, batch 256, L lognormal (mean 13500, sd 7600) clipped.
    4: Qwen3-8B shape, batch 32, L fixed at 65536 or 131072, k and s swept.
    """
    base = {
        0: dict(name="single-request L2048 h16/8", model="qwen3-1.7b", batch=1,
                lengths=("fixed", 2048), k=8, s=0.05),
        1: dict(name="qwen3-1.7b-shape B64 L~U[4K,16K]", model="qwen3-1.7b", batch=64,
                lengths=("uniform", 4096, 16384), k=8, s=0.05),
        2: dict(name="qwen3-8b-shape B128 L~lognormal(12K,7.6K)", model="qwen3-8b",
                batch=128, lengths=("lognormal", 12000.0, 7600.0, 1024, 32768), k=8, s=0.05),
        3: dict(name="qwen3-14b-shape B256 L~lognormal(13.5K,7.6K)", model="qwen3-14b",
                batch=256, lengths=("lognormal", 13500.0, 7600.0, 1024, 32768), k=8, s=0.05),
        4: dict(name="qwen3-8b-shape B32 L128K", model="qwen3-8b", batch=32,
                lengths=("fixed", 131072), k=8, s=0.05),
    }[index]
    base = dict(base)
    base.update(overrides)
    return base


def context_lengths(lengths: tuple, batch: int, rng: np.random.Generator) -> np.ndarray:
    """Draw the verify-time context length L of every request."""
    kind = lengths[0]
    if kind == "fixed":
        return np.full(batch, int(lengths[1]), dtype=np.int64)
    if kind == "uniform":
        lo, hi = int(lengths[1]), int(lengths[2])
        return rng.integers(lo, hi + 1, size=batch).astype(np.int64)
    if kind == "lognormal":
        mean, sd, lo, hi = float(lengths[1]), float(lengths[2]), int(lengths[3]), int(lengths[4])
        sigma2 = math.log1p((sd / mean) ** 2)
        mu = math.log(mean) - 0.5 * sigma2
        x = rng.lognormal(mu, math.sqrt(sigma2), size=batch)
        return np.clip(np.rint(x), lo, hi).astype(np.int64)
    raise ValueError(f"unknown length distribution {kind!r}")


def assign_buckets_least_loaded(batch: int, num_buckets: int) -> np.ndarray:
    """Greedy assignment of requests, in arrival order, to the least-loaded
    bucket (load = request count, ties to the lowest bucket id)."""
    load = np.zeros(num_buckets, dtype=np.int64)
    out = np.empty(batch, dtype=np.int32)
    for r in range(batch):
        b = int(np.argmin(load))  # argmin returns the first minimum
        out[r] = b
        load[b] += 1
    return out


def to_numpy_bf16(t: torch.Tensor) -> np.ndarray:
    """bfloat16 tensor -> numpy uint16 array of its bit patterns (host copy)."""
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)


@dataclass
class Workload:
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    k: int
    s: float
    sm_scale: float
    verify_lens: np.ndarray          # int64 [B]: L_r, context length at verify time
    caps: np.ndarray                 # int64 [B]: tokens written to the pages (L_r + k)
    bucket_ids: np.ndarray           # int32 [B]
    k_pages: torch.Tensor            # bf16 [num_pages][Hkv][page][d]
    v_pages: torch.Tensor            # bf16 [num_pages][Hkv][page][d]
    block_table: torch.Tensor        # int32 [B][bt_stride]
    qbank: torch.Tensor              # bf16 [B][2k+1][Hq][d]
    pillar_pos: List[np.ndarray] = field(default_factory=list)  # per request: int64 [Hkv][P]
    seed: int = 0
    device: str = "cpu"

    @property
    def batch(self) -> int:
        return int(self.verify_lens.shape[0])

    @property
    def num_pages(self) -> int:
        return int(self.k_pages.shape[0])

    @property
    def bt_stride(self) -> int:
        return int(self.block_table.shape[1])


def queries_per_request(is_verify: np.ndarray, k: int) -> np.ndarray:
    return np.where(is_verify, k + 1, 1).astype(np.int64)


def cycle_state(w: Workload, t: int):
    """State of launch t of the steady cycle (verify bucket = t mod (k+1)).

    A request of bucket b verifies at L_b when t = b; otherwise it is at
    draft step j = (t - b) mod (k+1) in [1, k] with context L + j, whose
    selection was taken at the verify (sel_len = L).
    Returns (verify_bucket, is_verify [B] bool, ctx_lens [B] int64,
    draft_step [B] int64 (0 for verify)).
    """
    kp1 = w.k + 1
    vb = t % kp1
    is_verify = w.bucket_ids == vb
    step = (vb - w.bucket_ids.astype(np.int64)) % kp1
    ctx = np.where(is_verify, w.verify_lens, w.verify_lens + step)
    return vb, is_verify, ctx.astype(np.int64), np.where(is_verify, 0, step)


def pack_rows(w: Workload, is_verify: np.ndarray, draft_step: np.ndarray,
              device: Optional[str] = None) -> torch.Tensor:
    """Pack the query rows of one unified launch in request order:
    k+1 rows for a verify request, one row for a draft request."""
    dev = device or w.device
    parts = []
    for r in range(w.batch):
        if is_verify[r]:
            parts.append(w.qbank[r, : w.k + 1])
        else:
            j = int(draft_step[r])
            parts.append(w.qbank[r, w.k + j: w.k + j + 1])
    return torch.cat(parts, 0).to(dev).contiguous()


def make_workload(spec: dict, seed: int, device: str = "cpu", *,
                  pillar_frac: float = 0.05, pillar_k_shift: float = 3.0,
                  q_shift: Optional[float] = None, head_dim: int = 128,
                  page_size: int = 16, lengths: Optional[np.ndarray] = None,
                  extra_pages: int = 0) -> Workload:
    """Build a seeded workload on `device` ("cpu" or "cuda")."""
    hq, hkv = ATTN_SHAPES[spec["model"]] if "model" in spec else (spec["hq"], spec["hkv"])
    hq = spec.get("hq", hq)
    hkv = spec.get("hkv", hkv)
    k, s = int(spec["k"]), float(spec["s"])
    d = head_dim
    if q_shift is None:
        q_shift = math.sqrt(d)
    rng = np.random.default_rng(np.random.SeedSequence(seed))
    B = int(spec["batch"])
    L = np.asarray(lengths, dtype=np.int64) if lengths is not None else \
        context_lengths(spec["lengths"], B, rng)
    B = int(L.shape[0])
    caps = L + k
    npages = (caps + page_size - 1) // page_size
    total = int(npages.sum()) + int(extra_pages)
    bt_stride = int(npages.max())

    gcpu = torch.Generator(device="cpu")
    gcpu.manual_seed(int(rng.integers(0, 2**62)))
    gdev = torch.Generator(device=device)
    gdev.manual_seed(int(rng.integers(0, 2**62)))

    perm = torch.randperm(total, generator=gcpu).to(torch.int32)
    block_table = torch.zeros(B, bt_stride, dtype=torch.int32)
    off = 0
    for r in range(B):
        block_table[r, : npages[r]] = perm[off: off + npages[r]]
        off += int(npages[r])

    k_pages = torch.zeros(total, hkv, page_size, d, dtype=torch.bfloat16, device=device)
    v_pages = torch.zeros_like(k_pages)
    qbank = torch.empty(B, 2 * k + 1, hq, d, dtype=torch.bfloat16, device=device)
    G = hq // hkv
    pillar_pos: List[np.ndarray] = []
    for r in range(B):
        cap, Lr, npr = int(caps[r]), int(L[r]), int(npages[r])
        kf = torch.randn(npr * page_size, hkv, d, generator=gdev, device=device)
        vf = torch.randn(npr * page_size, hkv, d, generator=gdev, device=device)
        kf[cap:] = 0.0
        vf[cap:] = 0.0
        u = torch.randn(hkv, d, generator=gdev, device=device)
        u = u / u.norm(dim=1, keepdim=True)
        P = int(round(pillar_frac * Lr))
        pos = np.stack([torch.randperm(Lr, generator=gcpu)[:P].numpy() for _ in range(hkv)]) \
            if P > 0 else np.zeros((hkv, 0), dtype=np.int64)
        pillar_pos.append(pos.astype(np.int64))
        if P > 0:
            pos_t = torch.as_tensor(pos, device=device)
            for h in range(hkv):
                kf[pos_t[h], h, :] += pillar_k_shift * u[h]
        phys = block_table[r, :npr].to(device=device, dtype=torch.long)
        k_pages[phys] = kf.view(npr, page_size, hkv, d).permute(0, 2, 1, 3).to(torch.bfloat16)
        v_pages[phys] = vf.view(npr, page_size, hkv, d).permute(0, 2, 1, 3).to(torch.bfloat16)
        qf = torch.randn(2 * k + 1, hq, d, generator=gdev, device=device)
        qf += q_shift * u.repeat_interleave(G, dim=0)[None, :, :]
        qbank[r] = qf.to(torch.bfloat16)

    buckets = assign_buckets_least_loaded(B, k + 1)
    return Workload(num_q_heads=hq, num_kv_heads=hkv, head_dim=d, page_size=page_size,
                    k=k, s=s, sm_scale=1.0 / math.sqrt(d), verify_lens=L, caps=caps,
                    bucket_ids=buckets, k_pages=k_pages, v_pages=v_pages,
                    block_table=block_table.to(device), qbank=qbank,
                    pillar_pos=pillar_pos, seed=seed, device=device)

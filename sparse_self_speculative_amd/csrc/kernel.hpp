// The persistent SparseSpec kernel [talk notes "Accelerating Large-Scale
// Reasoning Model Inference with Sparse Self-Speculative Decoding", sections
// PillarAttn (paper §4.1) and Unified batch scheduler (paper §4.2, §5.6
// Fig. 15)].
//
// One kernel serves every entry point.  Each work-group is resident for the
// whole launch (one per CU), and each of its WAVES waves is an independent
// worker with its own LDS region; after a short prologue that derives the
// task schedule, no wave ever waits at a work-group barrier.
//
// Tasks (one wave each):
//   verify chunk  cp pages of one (item, KV head): full attention of the
//                 k+1 queries x G heads, logits dumped (cp is chosen per
//                 launch, see verify_chunk_pages);
//   score chunk   kScoreChunk keys of one (item, KV head): PillarAttn scores
//                 from the dump;
//   draft chunk   up to kDraftChunk positions of one (item, KV head)'s token
//                 set (an item's chunks are of equal length).
// Static tasks come from one queue (split over the XCDs): verify chunks
// (longest contexts first), then (selection-only launches) score chunks,
// then draft chunks (longest chunks first).  Whichever wave finishes the last chunk of an
// (item, KV head) merges the chunk partials; in a unified launch it then
// publishes that (item, KV head)'s score chunks on a second list, which
// every wave serves before the static queue, and whichever wave scores the
// last chunk runs the Top-K selection.  So the selection of a long context
// starts as soon as its verify ends, while drafts still stream.
//
// Cross-work-group data (partials, the dump, LSE, scores, histograms) uses
// device-coherent accesses and relaxed atomics (see sspec_common.hpp); no
// L2 write-back or invalidate is ever issued.
#pragma once

#include <hip/hip_runtime.h>

#include <array>
#include <cstdint>

#include "draft.hpp"
#include "select.hpp"
#include "sspec_common.hpp"
#include "verify.hpp"

// SSPEC_ONLY_NQT (compile-time, development builds only) restricts the
// instantiated kernels to one query-tile count to shorten compiles.
#ifndef SSPEC_ONLY_NQT
#define SSPEC_ONLY_NQT 0
#endif

namespace sspec {

constexpr int kLdsMax = 160 * 1024;
constexpr uint32_t kSpinLimit = 1u << 18;
#ifndef SSPEC_FAR_WAIT
#define SSPEC_FAR_WAIT 3000
#endif
constexpr int kFarWait = SSPEC_FAR_WAIT;   // 100 MHz ticks

struct Job {
  int mode;
  int naive;                   // unified: naive batching (every item in the verify's tile shape)
  sspec_paged_kv kv;
  const uint16_t* q;
  const int32_t* seq_ids;      // null: item i is request i
  const int32_t* ctx_lens;
  const int32_t* bucket_ids;   // unified
  int verify_bucket;
  int n;                       // items of this launch
  int layout_n;                // items the workspace layout is carved for (the same for
                               // every launch of one call)
  int num_seqs;                // valid request ids are [0, num_seqs)
  int max_verify, max_ctx, hq, hkv, k;
  double s;
  float scale;
  float* logits;               // verify: dump written; topk: dump read
  const float* lse_in;         // topk: LSE read
  int64_t lstride;             // row stride of `logits`
  int32_t* sel_idx;
  int sel_stride;
  int32_t* sel_count;
  int32_t* sel_len;
  uint16_t* out;
  float* lse;
  uint8_t* ws;
  size_t ws_bytes;   // workspace size the host checked against its layout
};

// Kinds of items, in schedule order.
constexpr int kKindVerify = 0, kKindScore = 1, kKindDraft = 2, kKindNone = 3;

__device__ __forceinline__ bool ctx_ok(int L, int max_ctx, const sspec_paged_kv& kv) {
  return L >= 1 && L <= max_ctx && (int64_t)L <= (int64_t)kv.bt_stride * kPage;
}

// ------------------------------------------------------------------ LDS ---
constexpr int kSchedBytes =
    (int)align256(2 * kMaxItems + 2 * kMaxItems + 4 * (kMaxItems + 1) + 4 * 16 + 4 * 16 + 4 * 2 * kShards);

__host__ __device__ constexpr int cmax(int a, int b) { return a > b ? a : b; }

template <int NQT>
struct WaveLdsBytes {
  static constexpr int raw = cmax(cmax(VerifyWaveLds<NQT>::kBytes, DraftWaveLds::kBytes), SelectWaveLds::kBytes);
  static constexpr int value = (raw + 255) / 256 * 256;
};

template <int NQT>
constexpr int waves_for() {
  const int w = (kLdsMax - kSchedBytes) / WaveLdsBytes<NQT>::value;
  return w > 4 ? 4 : w;
}

template <int NQT, int WAVES>
struct KernelLds {
  static constexpr int kPerWave = WaveLdsBytes<NQT>::value;
  static constexpr int kWaveOff = kSchedBytes;
  static constexpr int kBytes = kWaveOff + WAVES * kPerWave;
  static_assert(kBytes <= kLdsMax, "LDS budget");
  // prologue temporaries live in the (not yet used) wave regions
  static_assert(3 * kMaxItems * 4 <= WAVES * kPerWave, "prologue scratch");
};

// Exclusive scan over the work-group (WAVES waves); *total gets the sum.
template <int WAVES>
__device__ __forceinline__ int block_excl_scan(int v, int* tmp, int* total) {
  const int wave = threadIdx.x >> 6;
  int wt;
  const int x = wave_excl_scan(v, &wt);
  if (lane_id() == 0) tmp[wave] = wt;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < WAVES; ++w) {
    const int t = tmp[w];
    base += (w < wave) ? t : 0;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return base + x;
}

// Work-group sums (or maxima) of K per-thread values, in place: every
// thread gets the totals.  One barrier round; red holds WAVES*K ints.
template <int WAVES, int K, bool MAX>
__device__ __forceinline__ void block_sums(int (&v)[K], int* red) {
  const int wave = threadIdx.x >> 6;
#pragma unroll
  for (int k = 0; k < K; ++k) v[k] = MAX ? wave_max_i(v[k]) : wave_sum_i(v[k]);
  if (lane_id() == 0) {
#pragma unroll
    for (int k = 0; k < K; ++k) red[wave * K + k] = v[k];
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < K; ++k) {
    int t = red[k];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) t = MAX ? max(t, red[w * K + k]) : t + red[w * K + k];
    v[k] = t;
  }
  __syncthreads();   // red may be reused
}

__device__ __forceinline__ int find_owner(const int* pre, int n, int t) {
  // largest p in [0, n) with pre[p] <= t  (pre non-decreasing, pre[0] = 0)
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (pre[mid] <= t) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// Draft-set geometry of request r, with the selection state clamped so that
// the set never exceeds max_ctx positions: n_sel <= sel_stride,
// sel_len in [0, max_ctx], n_sel <= sel_len.  The last cut is exact for an
// ascending row of distinct indices: once a rollback has lowered sel_len,
// the entries past the first sel_len can only hold indices >= sel_len,
// which the draft leaves out anyway.  `clamped` reports bad state only (a
// count outside [0, sel_stride], a length outside [0, max_ctx]).
struct DraftGeom {
  int n_sel, sel_len, N;
  bool clamped;
};
__device__ __forceinline__ DraftGeom draft_geom_of(const Job& p, int n0, int s0, int L) {
  DraftGeom g;
  g.sel_len = s0 < 0 ? 0 : (s0 > p.max_ctx ? p.max_ctx : s0);
  const int n = n0 < 0 ? 0 : (n0 > p.sel_stride ? p.sel_stride : n0);
  g.n_sel = n > g.sel_len ? g.sel_len : n;
  g.clamped = n != n0 || g.sel_len != s0;
  g.N = draft_set_size(g.n_sel, g.sel_len, L);
  return g;
}
__device__ __forceinline__ DraftGeom draft_geom(const Job& p, int r, int L) {
  return draft_geom_of(p, p.sel_count[r], p.sel_len[r], L);
}

// -------------------------------------------------------------- kernel ---
template <int G, int NQT, int WAVES>
__global__ __launch_bounds__(WAVES * kWave) void sspec_kernel(Job p) {
  using Lds = KernelLds<NQT, WAVES>;
  __shared__ __align__(256) char lds[Lds::kBytes];
  int16_t* s_order = reinterpret_cast<int16_t*>(lds);      // [kMaxItems] item | kind << 12, schedule order
  int16_t* s_vb = s_order + kMaxItems;                       // [kMaxItems] verify requests before item i
  int* s_pref = reinterpret_cast<int*>(s_vb + kMaxItems);    // [kMaxItems + 1] static task prefix
  int* s_misc = s_pref + kMaxItems + 1;                      // [16]
  int* s_tmp = s_misc + 16;                                  // [16] scan scratch
  int* s_lt = s_tmp + 16;                                    // [kShards] score tasks per shard list
  int* s_loff = s_lt + kShards;                              // [kShards] first entry of each list
  uint32_t* t_key = reinterpret_cast<uint32_t*>(lds + Lds::kWaveOff);  // prologue only
  int* t_cnt = reinterpret_cast<int*>(t_key + kMaxItems);
  int* t_pos = t_cnt + kMaxItems;
  int* s_red = t_pos + kMaxItems;                            // [WAVES][16] reduction scratch

  const uint64_t t_entry = SSPEC_TRACE ? __builtin_amdgcn_s_memrealtime() : 0;
  uint64_t t_ph[kTrPhases] = {};   // prologue phase ends (trace builds)
#define SSPEC_PHASE(k) \
  if (SSPEC_TRACE) t_ph[k] = __builtin_amdgcn_s_memrealtime();
  WsHeader* hdr = reinterpret_cast<WsHeader*>(p.ws);
  uint32_t* err = &hdr->err;
  const int n = p.n, hkv = p.hkv, kp1 = p.k + 1, M = G * kp1;
  const int mp = round_up((p.hq / hkv) * kp1, 4);   // dump row pitch
  const bool uni = p.mode == kModeUnified;
  const bool reporter = blockIdx.x == 0;
  const bool sel_only = p.mode == kModeTopk;
  const int skeys = sel_only ? kScoreChunkSel : kScoreChunk;   // keys per score task
  // score tasks of a context of L keys (two constant divisors)
  auto nscore = [&](int L) __attribute__((always_inline)) {
    return sel_only ? score_splits(L, kScoreChunkSel) : score_splits(L, kScoreChunk);
  };
  const WsLayout wl(p.mode, p.layout_n, p.max_verify, p.max_ctx, p.hq, hkv, p.k);
  if (wl.total > p.ws_bytes || n > p.layout_n) {
    // the host sized the workspace with another layout (objects of
    // differently configured builds linked together): touch nothing
    if (reporter && threadIdx.x == 0) set_error(err, SSPEC_DEV_ERR_LAYOUT);
    return;
  }
  // ---------------- prologue: every work-group derives the same schedule
  // Items are dealt round-robin (item i = tid + e*kThr), so every wave takes
  // a share; per-item results are summed in registers and reduced over the
  // work-group a few values at a time (block_sums), one barrier per round.
  constexpr int kThr = WAVES * kWave;
  constexpr int IPT = (kMaxItems + kThr - 1) / kThr;
  const int tid = threadIdx.x;
  // every per-item input in one round of loads, issued before the
  // workspace check so that the two memory round trips overlap
  int rr[IPT], Lr[IPT], scn[IPT], sln[IPT], isv[IPT];
#pragma unroll
  for (int e = 0; e < IPT; ++e) {
    const int i = tid + e * kThr;
    rr[e] = -1;
    if (i < n) rr[e] = p.seq_ids ? p.seq_ids[i] : i;
  }
#pragma unroll
  for (int e = 0; e < IPT; ++e) {
    const int i = tid + e * kThr;
    const bool ok = rr[e] >= 0 && rr[e] < p.num_seqs;
    Lr[e] = ok ? p.ctx_lens[rr[e]] : 0;
    scn[e] = (ok && p.sel_count) ? p.sel_count[rr[e]] : 0;
    sln[e] = (ok && p.sel_len) ? p.sel_len[rr[e]] : 0;
    isv[e] = (i < n && uni) ? (p.bucket_ids[i] == p.verify_bucket) : 0;
  }
  // The zero-state zone of this layout must read zero (see WsLayout): the
  // workspace was initialised, and no aborted launch or call with another
  // layout left state in it that the host did not clear.  Every work-group
  // reads the same value (only work-group 0 lowers it, and never below this
  // launch's zone_end), so all of them take the same branch.
  if (threadIdx.x == 0) {
    const uint32_t mg = ld_coh_u(&hdr->magic);
    const uint64_t ce = __hip_atomic_load(&hdr->clean_end, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool ok = mg == kWsMagic && ce >= (uint64_t)wl.zone_end;
    if (reporter) {
      if (ok) __hip_atomic_store(&hdr->clean_end, (uint64_t)wl.zone_end, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else set_error(err, SSPEC_DEV_ERR_WS_STATE);
    }
    *reinterpret_cast<volatile int*>(lds) = ok;
  }
  __syncthreads();
  if (!*reinterpret_cast<volatile int*>(lds)) return;
  __syncthreads();   // the flag's LDS word is reused below
  SSPEC_PHASE(0)

  if (SSPEC_TRACE) {
    __builtin_amdgcn_s_waitcnt(0);   // the stamp includes the loads' latency
    SSPEC_PHASE(1)
  }
  // verify requests before item i: scans of the rounds' flags, three rounds
  // per scan packed in 10-bit fields (each round has at most kThr <= 1023)
  int vbr[IPT];
  {
    int carry = 0;
#pragma unroll
    for (int e0 = 0; e0 < IPT; e0 += 3) {
      int packed = 0;
#pragma unroll
      for (int e = e0; e < IPT && e < e0 + 3; ++e) packed |= isv[e] << (10 * (e - e0));
      int tot;
      const int pre = block_excl_scan<WAVES>(packed, s_tmp, &tot);
#pragma unroll
      for (int e = e0; e < IPT && e < e0 + 3; ++e) {
        const int i = tid + e * kThr;
        vbr[e] = carry + ((pre >> (10 * (e - e0))) & 1023);
        carry += (tot >> (10 * (e - e0))) & 1023;
        if (i < kMaxItems) s_vb[i] = (int16_t)vbr[e];
      }
    }
  }
  SSPEC_PHASE(2)
  // per-thread sums: [0] verify pages (per KV head), [1] verify items,
  // [2] published score tasks, [3 + x] score tasks on list x; and the
  // longest verify context
  int acc[11], lmx[1] = {0};
#pragma unroll
  for (int k = 0; k < 11; ++k) acc[k] = 0;
  // tasks that pair (i, h) publishes, per_pair for each h, counted on the
  // pair's list (i*hkv + h) % kShards
  auto add_list_tasks = [&](int i, int per_pair) __attribute__((always_inline)) {
    acc[2] += hkv * per_pair;
#pragma unroll
    for (int x = 0; x < kShards; ++x) {
      const int h0 = ((x - i * hkv) % kShards + kShards) % kShards;   // first h with (i*hkv+h)%8 == x
      acc[3 + x] += h0 < hkv ? per_pair * ((hkv - h0 + kShards - 1) / kShards) : 0;
    }
  };
  bool vk[IPT];
  int dk[IPT];   // naive batching: draft set size (its task count needs the chunk length)
#pragma unroll
  for (int e = 0; e < IPT; ++e) {
    const int i = tid + e * kThr;
    vk[e] = false;
    dk[e] = -1;
    if (i >= n) {
      if (i < round_up(n, 32)) t_key[i] = 0xffffffffu;   // padding: ranks after every item
      continue;
    }
    int kind = kKindNone, size = 0, cnt = 0;
    const int r = rr[e];
    if (r < 0 || r >= p.num_seqs) {
      if (reporter) set_error(err, SSPEC_DEV_ERR_SEQ_RANGE);
    } else {
      const int L = Lr[e];
      const bool verify_like = p.mode == kModeVerify || (uni && isv[e]);
      if (verify_like || p.mode == kModeTopk) {
        const bool okc = p.mode == kModeTopk ? (L >= 1 && L <= p.max_ctx) : ctx_ok(L, p.max_ctx, p.kv);
        if (!okc) {
          if (reporter) set_error(err, SSPEC_DEV_ERR_CTX_RANGE);
        } else if (L < kp1) {
          if (reporter) set_error(err, SSPEC_DEV_ERR_VERIFY_SHORT);
        } else if (uni && vbr[e] >= p.max_verify) {
          if (reporter) set_error(err, SSPEC_DEV_ERR_TOO_MANY_VERIFY);
        } else if (p.mode == kModeTopk) {
          kind = kKindScore;
          size = L;
          cnt = hkv * nscore(L);
        } else {
          kind = kKindVerify;
          size = L;
          vk[e] = true;   // task count set once the chunk length is known
          acc[0] += cdiv(L, kPage);
          acc[1] += 1;
          lmx[0] = max(lmx[0], L);
          // pair (i, h) publishes its score chunks on list (i*hkv + h) % kShards
          if (uni) add_list_tasks(i, nscore(L));
        }
      } else {
        if (!ctx_ok(L, p.max_ctx, p.kv)) {
          if (reporter) set_error(err, SSPEC_DEV_ERR_CTX_RANGE);
        } else {
          const DraftGeom dg = draft_geom_of(p, scn[e], sln[e], L);
          if (dg.clamped && reporter) set_error(err, SSPEC_DEV_ERR_SEL_RANGE);
          kind = kKindDraft;
          if (p.naive) {
            dk[e] = dg.N;
            size = dg.N;
          } else {
            const int ns = draft_splits(dg.N);
            cnt = hkv * ns;
            size = cdiv(dg.N, ns);   // chunk length: larger chunks go first
          }
        }
      }
    }
    // schedule key: kind first, then larger first (size <= kMaxCtx < 2^21),
    // then item order; for drafts the size is the chunk length, so the static
    // queue ends with the shortest tasks.  Keys are distinct.
    t_key[i] = ((uint32_t)kind << 30) | ((uint32_t)(0x1fffff - min(size, 0x1fffff)) << 9) | (uint32_t)i;
    t_cnt[i] = cnt;
  }
  SSPEC_PHASE(3)
  block_sums<WAVES, 11, false>(acc, s_red);
  block_sums<WAVES, 1, true>(lmx, s_red);
  SSPEC_PHASE(4)
  if (tid < kShards) {
    int o = 0;
#pragma unroll
    for (int x = 0; x < kShards; ++x) o += x < tid ? acc[3 + x] : 0;
    s_loff[tid] = o;
#pragma unroll
    for (int x = 0; x < kShards; ++x)
      if (x == tid) s_lt[tid] = acc[3 + x];
  }
  if (tid == 0) s_misc[1] = acc[2];
  // Verify chunk length of this launch (the same in every work-group).
  // Longer contexts get shorter chunks (verify_pair_chunk); the base length
  // is the shortest of cp0 * (1 + c/8), c = 0..3, that still gives every
  // verify chunk its own wave (c = 3 always does when cp0 does, as no chunk
  // is cut by more than a quarter); if none does, chunks stay at cp0.
  int cp, lmax;
  {
    const int W = (int)gridDim.x * WAVES;
    const int cp0 = verify_chunk_pages((int64_t)acc[0] * hkv, acc[1] * hkv, W);
    const int lm = lmx[0];
    int cand[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) cand[c] = 0;
    // (a launch without verify items, whose candidates are all 0, skips the
    // count and its reduction; acc[1] is the work-group's total)
    if (acc[1] > 0) {
#pragma unroll
      for (int e = 0; e < IPT; ++e) {
        if (!vk[e]) continue;
        const int f = verify_pair_frac(Lr[e], lm);
        const int pg = cdiv(Lr[e], kPage);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int cc = min(kVChunkMax, cp0 + (cp0 * c) / 8);
          cand[c] += hkv * cdiv_small(pg, verify_pair_chunk_f(cc, f));
        }
      }
      block_sums<WAVES, 4, false>(cand, s_red);
    }
    cp = cp0;
    lmax = 0;
#pragma unroll
    for (int c = 3; c >= 0; --c) {
      if (cand[c] <= W) {
        cp = min(kVChunkMax, cp0 + (cp0 * c) / 8);
        lmax = lm;
      }
    }
  }
  SSPEC_PHASE(5)
#pragma unroll
  for (int e = 0; e < IPT; ++e) {
    if (vk[e]) t_cnt[tid + e * kThr] = hkv * verify_splits(Lr[e], verify_pair_chunk(cp, Lr[e], lmax));
    if (dk[e] >= 0) t_cnt[tid + e * kThr] = hkv * naive_draft_splits(dk[e], cp);
  }
  SSPEC_PHASE(6)
  // rank = number of smaller keys; the keys are read 32 at a time (LDS
  // broadcast reads); t_key was written before the reductions' barriers,
  // t_cnt[i] by this thread
#pragma unroll
  for (int e = 0; e < IPT; ++e) {
    const int i = tid + e * kThr;
    if (i >= n) continue;
    const uint32_t ki = t_key[i];
    int rank = 0;
    for (int j0 = 0; j0 < n; j0 += 32) {
      u32x4 a[8];
#pragma unroll
      for (int g = 0; g < 8; ++g) a[g] = *reinterpret_cast<const u32x4*>(t_key + j0 + 4 * g);
#pragma unroll
      for (int g = 0; g < 8; ++g)
#pragma unroll
        for (int q = 0; q < 4; ++q) rank += (int)(a[g][q] < ki);
    }
    s_order[rank] = (int16_t)(i | ((ki >> 30) << 12));
    t_pos[rank] = t_cnt[i];
  }
  __syncthreads();
  SSPEC_PHASE(7)
  {
    int c[IPT], sum = 0;
#pragma unroll
    for (int e = 0; e < IPT; ++e) {
      const int q = tid * IPT + e;
      c[e] = q < n ? t_pos[q] : 0;
      sum += c[e];
    }
    int tot;
    int base = block_excl_scan<WAVES>(sum, s_tmp, &tot);
#pragma unroll
    for (int e = 0; e < IPT; ++e) {
      const int q = tid * IPT + e;
      if (q <= n && q <= kMaxItems) s_pref[q] = base;
      base += c[e];
    }
    if (tid == 0) {
      s_misc[0] = tot;
      s_misc[2] = tot;   // verify tasks, if every item verifies
      s_pref[n] = tot;
    }
  }
  __syncthreads();
  // static tasks [0, Tv) are verify chunks (items sorted first)
#pragma unroll
  for (int e = 0; e < IPT; ++e) {
    const int q = tid * IPT + e;
    if (q < n && (s_order[q] >> 12) != kKindVerify && (q == 0 || (s_order[q - 1] >> 12) == kKindVerify))
      s_misc[2] = s_pref[q];
  }
  __syncthreads();   // the wave regions (prologue scratch) are free from here on
  SSPEC_PHASE(8)
#undef SSPEC_PHASE
  const int T = s_misc[0];

  // ---------------- per-wave workers
  const int wave = threadIdx.x >> 6;
  const int lane = (int)lane_id();
  char* wlds = lds + Lds::kWaveOff + wave * Lds::kPerWave;
  uint32_t* vcount = reinterpret_cast<uint32_t*>(p.ws + wl.vcount);
  uint32_t* scount = reinterpret_cast<uint32_t*>(p.ws + wl.scount);
  uint32_t* dcount = reinterpret_cast<uint32_t*>(p.ws + wl.dcount);
  uint32_t* slist = reinterpret_cast<uint32_t*>(p.ws + wl.slist);
  uint32_t* ghist = reinterpret_cast<uint32_t*>(p.ws + wl.ghist);
  float* wdump = reinterpret_cast<float*>(p.ws + wl.dump);
  float* wscores = reinterpret_cast<float*>(p.ws + wl.scores);
  uint16_t* wtops = reinterpret_cast<uint16_t*>(p.ws + wl.tops);
  float* vparts = reinterpret_cast<float*>(p.ws + wl.vparts);
  uint32_t* selbits = reinterpret_cast<uint32_t*>(p.ws + wl.selbits);
  float* dparts = reinterpret_cast<float*>(p.ws + wl.dparts);

  // task trace (development builds)
  TraceRec* trace_buf = reinterpret_cast<TraceRec*>(p.ws + wl.trace);
  const uint32_t worker = blockIdx.x * WAVES + wave;
  // each worker owns kTraceRecords / 1024 record slots (no shared counter);
  // the reader clears them before the launch
  uint32_t trace_n = 0;
  auto trace = [&](uint32_t kind, int item, int h, int chunk, uint64_t t0, uint64_t t1 = 0) __attribute__((always_inline)) {
    if (!SSPEC_TRACE) return;
    if (t1 == 0) t1 = __builtin_amdgcn_s_memrealtime();
    constexpr uint32_t per = (uint32_t)(kTraceRecords / 1024);
    const uint32_t k = worker * per + trace_n;
    if (trace_n < per) ++trace_n;
    if (lane == 0) {
      if (k < kTraceRecords && k < (worker + 1) * per) {
        TraceRec r;
        r.t0 = t0;
        r.t1 = t1;
        r.kind_worker = kind | (worker << 8);
        r.item = (uint32_t)item;
        r.h = (uint32_t)h;
        r.chunk = (uint32_t)chunk;
        trace_buf[k] = r;
      }
    }
  };
  auto now = [&]() __attribute__((always_inline)) -> uint64_t { return SSPEC_TRACE ? __builtin_amdgcn_s_memrealtime() : 0; };
  if (SSPEC_TRACE && blockIdx.x == 0 && wave == 0 && lane == 0) hdr->trace_off = (uint32_t)(wl.trace / 256);
  if (SSPEC_TRACE && wave == 0) {
    trace(kTrPrologue, blockIdx.x, 0, 0, t_entry);
    for (int k = 0; k < kTrPhases; ++k) trace(kTrPrologue + 1, blockIdx.x, 0, k, k ? t_ph[k - 1] : t_entry, t_ph[k]);
  }

  // item -> (request, slot, first q/out/lse row)
  auto item_rows = [&](int i, int& r, int& slot, int& qrow) __attribute__((always_inline)) {
    r = p.seq_ids ? p.seq_ids[i] : i;
    if (uni) {
      slot = s_vb[i];
      qrow = i + p.k * s_vb[i];
    } else {
      slot = i;
      qrow = (p.mode == kModeDraft) ? i : i * kp1;
    }
  };

  // score-row geometry of (item i), shared by its score chunks and selection
  auto score_item = [&](int i, int& r, int& slot, int& L) __attribute__((always_inline)) -> ScoreItem {
    int qrow;
    item_rows(i, r, slot, qrow);
    L = p.ctx_lens[r];
    ScoreItem it;
    if (uni) {
      it.dump = wdump + (int64_t)slot * hkv * wl.lstride * mp;
      it.lstride = wl.lstride;
      it.lse = p.lse + (int64_t)qrow * p.hq;
    } else {
      it.dump = p.logits + (int64_t)i * hkv * p.lstride * mp;
      it.lstride = p.lstride;
      it.lse = p.lse_in + (int64_t)qrow * p.hq;
    }
    it.lse_row_stride = p.hq;
    it.kp1 = kp1;
    it.G = p.hq / hkv;   // runtime: a selection-only launch may run on any instance
    it.M = it.G * kp1;
    it.mp = round_up(it.M, 4);
    it.L = L;
    it.scores = wscores + (int64_t)slot * hkv * wl.sstride;
    it.tops = wtops + (int64_t)slot * hkv * wl.sstride;
    it.sstride = wl.sstride;
    it.chunk = skeys;
    it.hist = ghist + (int64_t)slot * hkv * kHistBins;
    return it;
  };

  // Publish the cnt score chunks of pair (i, h) on the pair's list, after
  // this wave's stores are complete (the caller drained them)
  auto publish = [&](int i, int h, int cnt) __attribute__((always_inline)) {
    const int x = (i * hkv + h) % kShards;
    uint32_t base = 0;
    if (lane == 0) base = __hip_atomic_fetch_add(hdr->sq_reserve(x), (uint32_t)cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    base = __builtin_amdgcn_readfirstlane(base) + (uint32_t)s_loff[x];
    for (int c = lane; c < cnt; c += kWave)
      if ((int)base + c < wl.nslist)
        st_coh_u(slist + (int64_t)(base + c) * kSlistStride, (((uint32_t)i * hkv + h) << 10 | (uint32_t)c) + 1u);
  };

  // score chunk c of (item i, KV head h); the last chunk starts the selection
  auto run_score = [&](int i, int h, int c) __attribute__((always_inline)) {
    int r, slot, L;
    const ScoreItem it = score_item(i, r, slot, L);
    uint64_t t0 = now();
    score_wave_chunk(it, h, c, wlds);
    trace(kTrScore, i, h, c, t0);
    const int64_t pair = (int64_t)slot * hkv + h;
    uint32_t* cnt = scount + pair;
    const int nc = nscore(L);
    t0 = now();
    const bool last_chunk = wave_arrive_last(cnt, (uint32_t)nc);
    trace(kTrArrive, i, h, c, t0);
    if (!last_chunk) return;
    if (lane == 0) st_coh_u(cnt, 0u);
    t0 = now();
    // the histogram is complete: bitmap selection (or its fallback)
    const int K = select_count(L, p.s);
    int32_t* sel = p.sel_idx + ((int64_t)r * hkv + h) * p.sel_stride;
    const float* srow = it.scores + (int64_t)h * it.sstride;
    const SelInfo info = select_prepare(it.hist + (int64_t)h * kHistBins, K, wlds);
    trace(kTrSelPrep, i, h, info.fallback, t0);
    if (info.fallback) {
      select_wave(srow, L, K, it.hist + (int64_t)h * kHistBins, sel, wlds, hdr->sel_path);
    } else {
      uint32_t* bits = selbits + pair * (wl.sstride / 16);
      const uint64_t t1 = now();
      collect_bits(it.tops + (int64_t)h * it.sstride, L, info.b1, bits);
      trace(kTrCollect, i, h, nc, t1);
      select_final(srow, L, K, info, bits, sel, wlds);
      if (lane == 0) __hip_atomic_fetch_add(hdr->sel_path + 0, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (h == 0 && lane == 0) {
      p.sel_count[r] = K;
      p.sel_len[r] = L;
    }
    trace(kTrSelect, i, h, L, t0);
  };

  auto run_verify = [&](int i, int local) __attribute__((always_inline)) {
    int r, slot, qrow;
    item_rows(i, r, slot, qrow);
    const int L = p.ctx_lens[r];
    const int cpi = verify_pair_chunk(cp, L, lmax);
    const int ns = verify_splits(L, cpi);
    const int h = local / ns, split = local - (local / ns) * ns;
    VerifyItem it;
    it.kp = p.kv.k_pages;
    it.vp = p.kv.v_pages;
    it.bt = p.kv.block_table + (int64_t)r * p.kv.bt_stride;
    it.num_pages = p.kv.num_pages;
    it.hkv = hkv;
    it.hq = p.hq;
    it.kp1 = kp1;
    it.G = G;
    it.M = M;
    it.L = L;
    it.scale = p.scale;
    it.q = p.q + (int64_t)qrow * p.hq * kD;
    it.q_row_stride = (int64_t)p.hq * kD;
    if (uni) {
      it.dump = wdump + (int64_t)slot * hkv * wl.lstride * mp;
      it.lstride = wl.lstride;
    } else {
      it.dump = p.logits + (int64_t)i * hkv * p.lstride * mp;
      it.lstride = p.lstride;
    }
    it.mp = mp;
    it.out = p.out + (int64_t)qrow * p.hq * kD;
    it.out_row_stride = (int64_t)p.hq * kD;
    it.lse = p.lse + (int64_t)qrow * p.hq;
    it.lse_row_stride = p.hq;
    it.err = err;
    bool done = false;
    uint64_t t0 = now();
    if (ns == 1) {
      verify_wave_chunk<NQT>(it, h, 0, cpi, nullptr, wlds);
      trace(kTrVerify, i, h, 0, t0);
      done = true;
    } else {
      float* parts = vparts + ((int64_t)slot * hkv + h) * wl.vsplits * part_split_floats(M);
      verify_wave_chunk<NQT>(it, h, split, cpi, parts + (int64_t)split * part_split_floats(M), wlds);
      trace(kTrVerify, i, h, split, t0);
      uint32_t* cnt = vcount + (int64_t)slot * hkv + h;
      t0 = now();
      const bool last_split = wave_arrive_last(cnt, (uint32_t)ns);
      trace(kTrArrive + 1, i, h, split, t0);
      if (last_split) {
        if (lane == 0) st_coh_u(cnt, 0u);
        t0 = now();
        verify_wave_lse(it, h, parts, ns);
        trace(kTrVCombine, i, h, ns, t0);
        done = true;
      }
    }
    if (done && uni) {
      // publish the score chunks of (i, h): LSE and dump are complete
      drain_vm();
      publish(i, h, nscore(L));
    }
    if (done && ns > 1) {
      // the output merge is off the selection's critical path
      t0 = now();
      verify_wave_out(it, h, vparts + ((int64_t)slot * hkv + h) * wl.vsplits * part_split_floats(M), ns);
      trace(kTrVCombine, i, h, -ns, t0);
    }
  };

  auto run_draft = [&](int i, int local) __attribute__((always_inline)) {
    int r, slot, qrow;
    item_rows(i, r, slot, qrow);
    const int L = p.ctx_lens[r];
    const DraftGeom dg = draft_geom(p, r, L);
    const int ns = p.naive ? naive_draft_splits(dg.N, cp) : draft_splits(dg.N);
    const int h = local / ns, split = local - (local / ns) * ns;
    DraftItem it;
    it.kp = p.kv.k_pages;
    it.vp = p.kv.v_pages;
    it.bt = p.kv.block_table + (int64_t)r * p.kv.bt_stride;
    it.num_pages = p.kv.num_pages;
    it.hkv = hkv;
    it.hq = p.hq;
    it.G = G;
    it.scale = p.scale;
    it.q = p.q + (int64_t)qrow * p.hq * kD;
    it.sel = p.sel_idx + (int64_t)r * hkv * p.sel_stride;
    it.sel_stride = p.sel_stride;
    it.n_sel = dg.n_sel;
    it.sel_len = dg.sel_len;
    it.L = L;
    it.ncols = p.hq / hkv;
    uint64_t wait_ticks = 0, phases[3] = {0, 0, 0};
    it.wait_ticks = SSPEC_TRACE ? &wait_ticks : nullptr;
    it.phases = SSPEC_TRACE ? phases : nullptr;
    it.out = p.out + (int64_t)qrow * p.hq * kD;
    it.lse = p.lse ? p.lse + (int64_t)qrow * p.hq : nullptr;
    it.err = err;
    // naive batching runs the draft in the verify's tile shape (the host
    // allows it only where the verify keeps its query tiles in registers)
    auto range = [&](int p0, int p1, float* part) __attribute__((always_inline)) {
      if constexpr (VerifyQ<NQT>::kRegs && NQT > 1) {
        if (p.naive) {
          draft_wave_range<G, NQT>(it, h, p0, p1, part, wlds);
          return;
        }
      }
      draft_wave_range<G>(it, h, p0, p1, part, wlds);
    };
    uint64_t t0 = now();
    if (ns == 1) {
      range(0, dg.N, nullptr);
      trace(kTrDraft, i, h, dg.N, t0);
      trace(kTrArrive + 2, i, h, (int)wait_ticks, t0);
      for (int k = 0; k < 3; ++k) trace(kTrArrive + 3 + k, i, h, (int)phases[k], t0);
      return;
    }
    // balanced chunks: [split*N/ns, (split+1)*N/ns), each <= kDraftChunk
    // (naive batching: <= the verify's chunk)
    const int p0 = (int)((int64_t)split * dg.N / ns), p1 = (int)((int64_t)(split + 1) * dg.N / ns);
    float* parts = dparts + ((int64_t)i * hkv + h) * wl.dsplits * part_split_floats(G);
    range(p0, p1, parts + (int64_t)split * part_split_floats(G));
    trace(kTrDraft, i, h, p1 - p0, t0);
    trace(kTrArrive + 2, i, h, (int)wait_ticks, t0);
    for (int k = 0; k < 3; ++k) trace(kTrArrive + 3 + k, i, h, (int)phases[k], t0);
    uint32_t* cnt = dcount + (int64_t)i * hkv + h;
    if (wave_arrive_last(cnt, (uint32_t)ns)) {
      if (lane == 0) st_coh_u(cnt, 0u);
      t0 = now();
      draft_wave_combine<G>(it, h, parts, ns);
      trace(kTrDCombine, i, h, ns, t0);
    }
  };

  // Scheduling.  The static tasks [0, T) are dealt round-robin to kShards
  // queues (task 8j + x is the j-th of queue x), and a wave claims from its
  // XCD's queue first, moving on to the next queue when one runs dry.  Every
  // task, the first included, is claimed by a running wave, so a launch
  // whose work-groups are not all resident at once (another kernel holds
  // some CUs) still runs every task: waves that start late find the queues
  // drained and leave.  Published score tasks go
  // to kShards lists (pair (i, h) to list (i*hkv + h) % kShards) and come
  // before static tasks.  They are claimed by ticket: a wave that sees
  // unclaimed entries on a list (head < reserve; reading the counters costs
  // a plain load), or that has nothing else left, takes ticket =
  // fetch_add(head) on it and owns that list entry.  An entry below the
  // reserve seen at the claim is being written by its publisher right now,
  // so the wave waits for it; an entry past it may be far off, so the wave
  // keeps serving static tasks meanwhile and, once the static queue is
  // drained, polls that entry alone.  A list's tickets past its total mean
  // every task on it has an owner.  A valid ticket is always published
  // eventually: the verifies that publish are all claimed and run by waves
  // that never wait.
  const uint32_t W = gridDim.x * (uint32_t)WAVES;
  const int home = (int)(blockIdx.x % kShards);
  int lt[kShards];
#pragma unroll
  for (int x = 0; x < kShards; ++x) lt[x] = s_lt[x];
  bool static_done = false, waiting = false, first = true;
  int qshift = 0;                          // static queues found empty (home first)
  uint32_t lists_left = uni ? (1u << kShards) - 1u : 0u;   // lists whose tickets are not all out
  int held = -1;          // owned score-list entry, not yet run
  bool held_soon = false; // the owned entry was reserved when claimed
  uint64_t held_t = 0;    // when an entry not yet reserved was claimed
  uint32_t polls = 0;
  uint64_t idle_t0 = 0;
  for (;;) {
    bool worked = false;
    if (lists_left != 0u && held < 0 && !first) {   // nothing is published before any work
      uint64_t hs = 0;
      if (lane < kShards) hs = __hip_atomic_load(&hdr->sq[lane].sq, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      // the first list, from this XCD's own on, with unclaimed published
      // entries: waves of different XCDs start on different lists, which
      // spreads claims made at the same moment (all waves picking the fullest
      // list would overshoot its reserve)
      int best = -1, any_left = -1;
      uint32_t best_rv = 0;
#pragma unroll
      for (int y = 0; y < kShards; ++y) {
        const int x = (home + y) % kShards;
        const uint64_t v = __shfl(hs, x);
        const uint32_t hd = __builtin_amdgcn_readfirstlane((uint32_t)v);
        const uint32_t rv = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
        if (!((lists_left >> x) & 1u)) continue;
        if (hd >= (uint32_t)lt[x]) {
          lists_left &= ~(1u << x);
          continue;
        }
        if (any_left < 0) any_left = x;
        if (rv > hd && best < 0) {
          best = x;
          best_rv = rv;
        }
      }
      if (best < 0 && static_done && any_left >= 0) {
        best = any_left;   // nothing else to do: own a future entry
        best_rv = 0;
      }
      if (best >= 0) {
        uint32_t tk = 0;
        if (lane == 0) tk = __hip_atomic_fetch_add(hdr->sq_head(best), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        tk = __builtin_amdgcn_readfirstlane(tk);
        if (tk < (uint32_t)s_lt[best] && s_loff[best] + (int)tk < wl.nslist) {
          held = s_loff[best] + (int)tk;
          held_soon = tk < best_rv;
          if (!held_soon) held_t = __builtin_amdgcn_s_memrealtime();
        } else {
          lists_left &= ~(1u << best);
        }
      }
    }
    if (held >= 0) {
      uint32_t e = 0;
      if (lane == 0) e = ld_coh_u(slist + (int64_t)held * kSlistStride);
      e = __builtin_amdgcn_readfirstlane(e);
      if (e != 0u) {
        if (lane == 0) st_coh_u(slist + (int64_t)held * kSlistStride, 0u);
        held = -1;
        e -= 1u;
        const int ih = (int)(e >> 10), c = (int)(e & 1023u);
        const int i = ih / hkv;
        // only this launch's publishers write entries: a verifying item and
        // one of its score chunks (anything else is stale state, never run)
        bool valid = i < n && p.bucket_ids[i] == p.verify_bucket && s_vb[i] < p.max_verify;
        if (valid) valid = c < nscore(p.ctx_lens[p.seq_ids ? p.seq_ids[i] : i]);
        if (valid) run_score(i, ih - i * hkv, c);
        else if (lane == 0) set_error(err, SSPEC_DEV_ERR_WS_STATE);
        worked = true;
      }
    }
    // an owned entry not yet reserved is usually published within a few
    // microseconds (the verifies end close together): poll it that long
    // before taking a static task, which may run for tens of microseconds
    const bool hold = held >= 0 && (held_soon || __builtin_amdgcn_s_memrealtime() - held_t < (uint64_t)kFarWait);
    if (!worked && !static_done && !hold) {
      const int qx = (home + qshift) % kShards;
      const uint64_t tc = now();
      uint32_t t = 0;
      if (lane == 0)
        t = kShards * __hip_atomic_fetch_add(&hdr->ctr[qx].queue_head, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + qx;
      t = __builtin_amdgcn_readfirstlane(t);
      if (first) trace(kTrPrologue + 2, (int)t, 0, 0, tc);   // the first claim
      first = false;
      if (t < (uint32_t)T) {
        const int g = (int)t;
        const int pos = find_owner(s_pref, n, g);
        const int oi = s_order[pos];
        const int i = oi & 0xfff, kind = oi >> 12;
        const int local = g - s_pref[pos];
        if (local < 0 || local >= s_pref[pos + 1] - s_pref[pos] || i >= n) {
          // cannot happen for a consistent schedule; never index with it
        } else if (kind == kKindVerify) run_verify(i, local);
        else if (kind == kKindDraft) run_draft(i, local);
        else if (kind == kKindScore) {
          int r, slot, qrow;
          item_rows(i, r, slot, qrow);
          const int nc = nscore(p.ctx_lens[r]);
          run_score(i, local / nc, local - (local / nc) * nc);
        }
        worked = true;
      } else if (++qshift == kShards) {
        static_done = true;   // every queue has run dry
      }
      if (!worked) continue;   // try the next queue
    }
    if (worked) {
      polls = 0;
      continue;
    }
    if (static_done && lists_left == 0u && held < 0) break;   // nothing left for this wave
    // waiting for a published score task (an owned entry or an unclaimed one)
    if (!waiting) {
      waiting = true;
      if (SSPEC_TRACE) idle_t0 = __builtin_amdgcn_s_memrealtime();
    }
    ++polls;
    if ((polls & 15u) == 0u && (ld_coh_u(err) & SSPEC_DEV_ERR_WAIT_TIMEOUT)) break;
    if (polls > kSpinLimit) {
      if (lane == 0) {
        set_error(err, SSPEC_DEV_ERR_WAIT_TIMEOUT);
        st_coh_u(&hdr->aborted, 1u);
      }
      break;
    }
    const uint32_t naps = polls < 8u ? 1u : (polls < 32u ? 4u : 16u);
    for (uint32_t z = 0; z < naps; ++z) __builtin_amdgcn_s_sleep(4);
  }
  if (SSPEC_TRACE && waiting) trace(kTrIdle, 0, 0, 0, idle_t0);

  // ---------------- exit: the last wave out of each shard reports it; the
  // last shard out resets every counter for the next launch
  drain_vm();
  if (lane == 0) {
    const uint32_t shard_waves = (gridDim.x - (uint32_t)home + kShards - 1) / kShards * (uint32_t)WAVES;
    const uint32_t nshards = gridDim.x < (uint32_t)kShards ? gridDim.x : (uint32_t)kShards;
    const uint32_t old = __hip_atomic_fetch_add(&hdr->ctr[home].exit_count, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old + 1u == shard_waves) {
      const uint32_t done = __hip_atomic_fetch_add(&hdr->exit_shards, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (done + 1u == nshards) {
        for (int x = 0; x < kShards; ++x) {
          st_coh_u(&hdr->ctr[x].queue_head, 0u);
          st_coh_u(&hdr->ctr[x].exit_count, 0u);
          st_coh_u(hdr->sq_head(x), 0u);
          st_coh_u(hdr->sq_reserve(x), 0u);
        }
        st_coh_u(&hdr->exit_shards, 0u);
        // a wave that gave up waiting left entries, counters or histograms
        // set: the zone is no longer known to be zero
        if (ld_coh_u(&hdr->aborted)) {
          __hip_atomic_store(&hdr->clean_end, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          st_coh_u(&hdr->aborted, 0u);
        }
      }
    }
  }
}

// ---- host side of the kernel table: one instance per (G, query tiles)
int fail(int code, const char* fmt, ...);
int check_launch(const char* what);
// resident work-groups of a kernel instance on the current device (cached)
int resident_grid(uint64_t key, const void* kernel, int threads, int* grid);

template <int G, int NQT>
int launch_kernel(const Job& p, hipStream_t st) {
  constexpr int WAVES = waves_for<NQT>();
  int grid = 0;
  const int rc = resident_grid((uint64_t)(G * 16 + NQT), reinterpret_cast<const void*>(&sspec_kernel<G, NQT, WAVES>),
                               WAVES * kWave, &grid);
  if (rc) return rc;
  hipLaunchKernelGGL((sspec_kernel<G, NQT, WAVES>), dim3(grid), dim3(WAVES * kWave), 0, st, p);
  return check_launch("sspec_kernel");
}
using KernelFn = int (*)(const Job&, hipStream_t);

template <int G, int NQT>
constexpr KernelFn kernel_entry() {
  if constexpr (NQT <= (G * (kMaxK + 1) + 15) / 16 && NQT <= kMaxRows / 16 &&
                (SSPEC_ONLY_NQT == 0 || SSPEC_ONLY_NQT == NQT))
    return &launch_kernel<G, NQT>;
  else return nullptr;
}
template <int G>
constexpr std::array<KernelFn, 8> kernel_row() {
  return {kernel_entry<G, 1>(), kernel_entry<G, 2>(), kernel_entry<G, 3>(), kernel_entry<G, 4>(),
          kernel_entry<G, 5>(), kernel_entry<G, 6>(), kernel_entry<G, 7>(), kernel_entry<G, 8>()};
}
// one table row per G, each built in its own translation unit
std::array<KernelFn, 8> kernel_table_row(int G);

#define SSPEC_STR2(x) #x
#define SSPEC_STR(x) SSPEC_STR2(x)
// The build macros that fix chunk sizes, waits, instances and the workspace
// layout, as one string: every object linked into one library must have
// been compiled with the same values (the host checks it before a launch).
inline const char* build_config() {
  return "vchunk_min=" SSPEC_STR(SSPEC_VCHUNK_MIN) " score_chunk=" SSPEC_STR(SSPEC_SCORE_CHUNK)
         " score_chunk_sel=" SSPEC_STR(SSPEC_SCORE_CHUNK_SEL) " draft_chunk=" SSPEC_STR(SSPEC_DRAFT_CHUNK) " vshort=" SSPEC_STR(SSPEC_VSHORT)
         " far_wait=" SSPEC_STR(SSPEC_FAR_WAIT)
         " trace=" SSPEC_STR(SSPEC_TRACE)
         " only_nqt=" SSPEC_STR(SSPEC_ONLY_NQT);
}

}  // namespace sspec

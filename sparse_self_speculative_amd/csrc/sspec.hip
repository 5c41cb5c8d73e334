// SparseSpec attention hot path for MI355X (gfx950): kernels and the C ABI
// declared in include/sspec.h.
//
// Method: talk notes "Accelerating Large-Scale Reasoning Model Inference
// with Sparse Self-Speculative Decoding" (MLSys 2026), sections PillarAttn
// (paper §4.1) and Unified batch scheduler (paper §4.2, §5.6 Fig. 15).
//
// Kernels
//   verify_kernel<NQT>   one work-group per (item, KV head, key chunk);
//                        the last chunk to finish merges the partials.
//   topk_kernel          one work-group per (item, KV head, score chunk);
//                        the last chunk to finish runs the radix select.
//   draft_kernel<G>      one work-group per (item, KV head, set chunk);
//                        the last chunk to finish merges the partials.
//   unified_kernel<G,NQT> persistent: one work-group per resident slot, all
//                        taking tasks from one atomic queue ordered
//                        [verify chunks][draft chunks][score chunks]; the
//                        verify merge, the selection and the draft merge are
//                        run by whichever work-group finishes a job's last
//                        part, so no work-group ever waits on a queue.  A
//                        score chunk waits (bounded) for its (request, KV
//                        head)'s LSE, which the verify merge publishes; every
//                        verify task is handed out before any score task and
//                        runs without waiting, so the wait always ends.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <array>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <unordered_map>

#include "draft.hpp"
#include "select.hpp"
#include "sspec_common.hpp"
#include "verify.hpp"

using namespace sspec;

// SSPEC_ONLY_G / SSPEC_ONLY_NQT (compile-time, development builds only)
// restrict the instantiated kernels to one shape to shorten compiles.
#ifndef SSPEC_ONLY_G
#define SSPEC_ONLY_G 0
#endif
#ifndef SSPEC_ONLY_NQT
#define SSPEC_ONLY_NQT 0
#endif

namespace {

// ------------------------------------------------------------ parameters ---
struct VerifyParams {
  sspec_paged_kv kv;
  const uint16_t* q;
  const int32_t* seq_ids;
  const int32_t* ctx_lens;
  int n, max_ctx, hq, k;
  float scale;
  uint16_t* out;
  float* lse;
  float* logits;
  int64_t lstride;
  uint8_t* ws;
  int vsplit_max;
};

struct TopkParams {
  const float* logits;
  const float* lse;
  int64_t lstride;
  const int32_t* seq_ids;
  const int32_t* ctx_lens;
  int n, num_seqs, max_ctx, hq, hkv, k;
  double s;
  int32_t* sel_idx;
  int sel_stride;
  int32_t* sel_count;
  int32_t* sel_len;
  uint8_t* ws;
  int ssplit_max;
};

struct DraftParams {
  sspec_paged_kv kv;
  const uint16_t* q;
  const int32_t* seq_ids;
  const int32_t* ctx_lens;
  const int32_t* sel_idx;
  int sel_stride;
  const int32_t* sel_count;
  const int32_t* sel_len;
  int n, max_ctx, hq;
  float scale;
  uint16_t* out;
  float* lse;
  uint8_t* ws;
};

struct UnifiedParams {
  sspec_paged_kv kv;
  const uint16_t* q;
  const int32_t* ctx_lens;
  const int32_t* bucket_ids;
  int verify_bucket, num_seqs, max_verify, max_ctx, hq, k;
  double s;
  float scale;
  int32_t* sel_idx;
  int sel_stride;
  int32_t* sel_count;
  int32_t* sel_len;
  uint16_t* out;
  float* lse;
  uint8_t* ws;
};

__device__ __forceinline__ bool ctx_ok(int L, int max_ctx, const sspec_paged_kv& kv) {
  return L >= 1 && L <= max_ctx && (int64_t)L <= (int64_t)kv.bt_stride * kPage;
}

// ------------------------------------------------------------ utilities ---
__global__ void zero_kernel(uint32_t* p, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

// ---------------------------------------------------------------- verify ---
template <int NQT>
__global__ __launch_bounds__(kThreads) void verify_kernel(VerifyParams p) {
  __shared__ __align__(16) char lds[VerifyLds<NQT>::kBytes];
  __shared__ int flag;
  const int hkv = p.kv.num_kv_heads;
  int b = blockIdx.x;
  const int split = b % p.vsplit_max;
  b /= p.vsplit_max;
  const int h = b % hkv, item = b / hkv;
  uint32_t* err = &reinterpret_cast<WsHeader*>(p.ws)->err;
  const int r = p.seq_ids[item];
  if (r < 0 || r >= p.kv.num_seqs) {
    if (split == 0 && h == 0 && threadIdx.x == 0) set_error(err, SSPEC_DEV_ERR_SEQ_RANGE);
    return;
  }
  const int L = p.ctx_lens[r];
  const int kp1 = p.k + 1;
  if (!ctx_ok(L, p.max_ctx, p.kv) || L < kp1) {
    if (split == 0 && h == 0 && threadIdx.x == 0)
      set_error(err, ctx_ok(L, p.max_ctx, p.kv) ? SSPEC_DEV_ERR_VERIFY_SHORT : SSPEC_DEV_ERR_CTX_RANGE);
    return;
  }
  const int ns = verify_splits(L);
  if (ns > p.vsplit_max) {  // cannot happen for L <= max_ctx; never index past the partials
    if (split == 0 && h == 0 && threadIdx.x == 0) set_error(err, SSPEC_DEV_ERR_CTX_RANGE);
    return;
  }
  if (split >= ns) return;
  const int G = p.hq / hkv, M = G * kp1;
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
  it.q = p.q + (int64_t)item * kp1 * p.hq * kD;
  it.q_row_stride = (int64_t)p.hq * kD;
  it.dump = p.logits + (int64_t)item * p.hq * kp1 * p.lstride;
  it.lstride = p.lstride;
  it.out = p.out + (int64_t)item * kp1 * p.hq * kD;
  it.out_row_stride = (int64_t)p.hq * kD;
  it.lse = p.lse + (int64_t)item * kp1 * p.hq;
  it.lse_row_stride = p.hq;
  it.err = err;
  if (ns == 1) {
    verify_chunk<NQT>(it, h, 0, nullptr, lds);
    return;
  }
  const VerifyWs wl(p.n, p.max_ctx, p.hq, hkv, p.k);
  float* parts = reinterpret_cast<float*>(p.ws + wl.parts) +
                 ((int64_t)item * hkv + h) * p.vsplit_max * M * kPartStride;
  verify_chunk<NQT>(it, h, split, parts + (int64_t)split * M * kPartStride, lds);
  uint32_t* cnt = reinterpret_cast<uint32_t*>(p.ws + wl.counters) + (int64_t)item * hkv + h;
  if (arrive_last(cnt, (uint32_t)ns, &flag)) {
    if (threadIdx.x == 0) atomic_store_agent(cnt, 0u);
    verify_combine(it, h, parts, ns);
  }
}

// ------------------------------------------------------------------ topk ---
__global__ __launch_bounds__(kThreads) void topk_kernel(TopkParams p) {
  __shared__ float lds[kSelectLdsFloats];
  __shared__ int flag;
  int b = blockIdx.x;
  const int c = b % p.ssplit_max;
  b /= p.ssplit_max;
  const int h = b % p.hkv, item = b / p.hkv;
  uint32_t* err = &reinterpret_cast<WsHeader*>(p.ws)->err;
  const int r = p.seq_ids[item];
  if (r < 0 || r >= p.num_seqs) {
    if (c == 0 && h == 0 && threadIdx.x == 0) set_error(err, SSPEC_DEV_ERR_SEQ_RANGE);
    return;
  }
  const int L = p.ctx_lens[r];
  const int kp1 = p.k + 1;
  if (L < 1 || L > p.max_ctx || L < kp1) {
    if (c == 0 && h == 0 && threadIdx.x == 0)
      set_error(err, (L >= 1 && L <= p.max_ctx) ? SSPEC_DEV_ERR_VERIFY_SHORT : SSPEC_DEV_ERR_CTX_RANGE);
    return;
  }
  const int ns = score_splits(L);
  if (ns > p.ssplit_max) {
    if (c == 0 && h == 0 && threadIdx.x == 0) set_error(err, SSPEC_DEV_ERR_CTX_RANGE);
    return;
  }
  if (c >= ns) return;
  const TopkWs wl(p.n, p.max_ctx, p.hkv);
  const int G = p.hq / p.hkv;
  ScoreItem it;
  it.dump = p.logits + (int64_t)item * p.hq * kp1 * p.lstride;
  it.lstride = p.lstride;
  it.lse = p.lse + (int64_t)item * kp1 * p.hq;
  it.lse_row_stride = p.hq;
  it.hq = p.hq;
  it.kp1 = kp1;
  it.G = G;
  it.M = G * kp1;
  it.L = L;
  it.scores = reinterpret_cast<float*>(p.ws + wl.scores) + (int64_t)item * p.hkv * wl.lstride;
  it.sstride = wl.lstride;
  score_chunk(it, h, c, lds);
  uint32_t* cnt = reinterpret_cast<uint32_t*>(p.ws + wl.counters) + (int64_t)item * p.hkv + h;
  if (arrive_last(cnt, (uint32_t)ns, &flag)) {
    if (threadIdx.x == 0) atomic_store_agent(cnt, 0u);
    const int K = select_count(L, p.s);
    select_topk(it.scores + (int64_t)h * it.sstride, L, K,
                p.sel_idx + ((int64_t)r * p.hkv + h) * p.sel_stride, lds);
    if (threadIdx.x == 0 && h == 0) {
      p.sel_count[r] = K;
      p.sel_len[r] = L;
    }
  }
}

// ----------------------------------------------------------------- draft ---
template <int G>
__device__ bool make_draft_item(DraftItem& it, const sspec_paged_kv& kv, int r, int L, int max_ctx,
                                const int32_t* sel_idx, int sel_stride, const int32_t* sel_count,
                                const int32_t* sel_len, const uint16_t* q, uint16_t* out, float* lse,
                                float scale, int hq, uint32_t* err, bool report) {
  if (!ctx_ok(L, max_ctx, kv)) {
    if (report) set_error(err, SSPEC_DEV_ERR_CTX_RANGE);
    return false;
  }
  // clamp the selection state so that the set never exceeds max_ctx
  // positions: n_sel <= sel_stride, sel_len in [0, max_ctx], n_sel <= sel_len
  int n_sel = sel_count[r];
  int sl = sel_len[r];
  const int sl_c = sl < 0 ? 0 : (sl > max_ctx ? max_ctx : sl);
  int n_c = n_sel < 0 ? 0 : (n_sel > sel_stride ? sel_stride : n_sel);
  n_c = n_c > sl_c ? sl_c : n_c;
  if (n_c != n_sel || sl_c != sl) {
    if (report) set_error(err, SSPEC_DEV_ERR_SEL_RANGE);
  }
  it.kp = kv.k_pages;
  it.vp = kv.v_pages;
  it.bt = kv.block_table + (int64_t)r * kv.bt_stride;
  it.num_pages = kv.num_pages;
  it.hkv = kv.num_kv_heads;
  it.hq = hq;
  it.G = G;
  it.scale = scale;
  it.q = q;
  it.sel = sel_idx + (int64_t)r * kv.num_kv_heads * sel_stride;
  it.sel_stride = sel_stride;
  it.n_sel = n_c;
  it.sel_len = sl_c;
  it.L = L;
  it.out = out;
  it.lse = lse;
  it.err = err;
  return true;
}

template <int G>
__global__ __launch_bounds__(kThreads) void draft_kernel(DraftParams p) {
  __shared__ __align__(16) char lds[DraftLds<G>::kBytes];
  const int hkv = p.kv.num_kv_heads;
  const int h = blockIdx.x % hkv, item = blockIdx.x / hkv;
  uint32_t* err = &reinterpret_cast<WsHeader*>(p.ws)->err;
  const int r = p.seq_ids[item];
  const bool report = h == 0 && threadIdx.x == 0;
  if (r < 0 || r >= p.kv.num_seqs) {
    if (report) set_error(err, SSPEC_DEV_ERR_SEQ_RANGE);
    return;
  }
  DraftItem it;
  if (!make_draft_item<G>(it, p.kv, r, p.ctx_lens[r], p.max_ctx, p.sel_idx, p.sel_stride, p.sel_count,
                          p.sel_len, p.q + (int64_t)item * p.hq * kD, p.out + (int64_t)item * p.hq * kD,
                          p.lse ? p.lse + (int64_t)item * p.hq : nullptr, p.scale, p.hq, err, report))
    return;
  // one work-group streams the whole set of its (item, KV head)
  draft_range<G>(it, h, 0, draft_set_size(it.n_sel, it.sel_len, it.L), nullptr, lds);
}

// --------------------------------------------------------------- unified ---
constexpr int kSchedInts = 5 * (kMaxSeqsUnified + 1) + 16 + kWaves;  // + misc [16] + scan scratch
constexpr uint32_t kSpinLimit = 1u << 18;

__device__ __forceinline__ int find_owner(const int* pre, int B, int t) {
  // largest r in [0, B) with pre[r] <= t  (pre is non-decreasing, pre[0] = 0)
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (pre[mid] <= t) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

template <int G, int NQT>
struct UnifiedLds {
  static constexpr int a = VerifyLds<NQT>::kBytes;
  static constexpr int b = DraftLds<G>::kBytes;
  static constexpr int c = kSelectLdsFloats * 4;
  static constexpr int ab = a > b ? a : b;
  static constexpr int kBytes = ab > c ? ab : c;
};

template <int G, int NQT>
__global__ __launch_bounds__(kThreads) void unified_kernel(UnifiedParams p) {
  __shared__ __align__(16) char lds[UnifiedLds<G, NQT>::kBytes];
  __shared__ int sched[kSchedInts];
  __shared__ int flag;
  WsHeader* hdr = reinterpret_cast<WsHeader*>(p.ws);
  uint32_t* err = &hdr->err;
  const int B = p.num_seqs, hkv = p.kv.num_kv_heads, kp1 = p.k + 1, M = G * kp1;
  const UnifiedWs wl(p.num_seqs, p.max_verify, p.max_ctx, p.hq, hkv, p.k);
  int* s_qoff = sched;                 // [B] first packed row of request r
  int* s_vslot = s_qoff + (kMaxSeqsUnified + 1);  // [B] verify slot or -1
  int* s_pv = s_vslot + (kMaxSeqsUnified + 1);    // [B+1] prefix of verify tasks
  int* s_pd = s_pv + (kMaxSeqsUnified + 1);       // [B+1] prefix of draft tasks
  int* s_ps = s_pd + (kMaxSeqsUnified + 1);       // [B+1] prefix of score tasks
  int* s_misc = s_ps + (kMaxSeqsUnified + 1);     // [16]
  int* tmp = sched + 5 * (kMaxSeqsUnified + 1) + 16;  // scan scratch [kWaves]
  const bool reporter = blockIdx.x == 0;

  // ---- prologue: every work-group derives the same schedule
  int isv[4], Ls[4], rows[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int r = 4 * threadIdx.x + e;
    isv[e] = 0;
    Ls[e] = 0;
    rows[e] = 0;
    if (r < B) {
      Ls[e] = p.ctx_lens[r];
      isv[e] = p.bucket_ids[r] == p.verify_bucket;
      rows[e] = isv[e] ? kp1 : 1;
    }
  }
  int tot;
  {
    const int v_in = isv[0] + isv[1] + isv[2] + isv[3];
    int vb = block_excl_scan(v_in, tmp, &tot);
    const int r_in = rows[0] + rows[1] + rows[2] + rows[3];
    int rb = block_excl_scan(r_in, tmp, &tot);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 4 * threadIdx.x + e;
      if (r < B) {
        s_qoff[r] = rb;
        s_vslot[r] = isv[e] ? vb : -1;
      }
      rb += rows[e];
      vb += isv[e];
    }
  }
  int cv[4], cd[4], cs[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int r = 4 * threadIdx.x + e;
    cv[e] = cd[e] = cs[e] = 0;
    if (r >= B) continue;
    const int L = Ls[e];
    const bool okc = ctx_ok(L, p.max_ctx, p.kv);
    if (!okc) {
      if (reporter) set_error(err, SSPEC_DEV_ERR_CTX_RANGE);
      continue;
    }
    if (isv[e]) {
      if (L < kp1) {
        if (reporter) set_error(err, SSPEC_DEV_ERR_VERIFY_SHORT);
        continue;
      }
      if (s_vslot[r] >= p.max_verify) {
        if (reporter) set_error(err, SSPEC_DEV_ERR_TOO_MANY_VERIFY);
        continue;
      }
      cv[e] = hkv * verify_splits(L);
      cs[e] = hkv * score_splits(L);
    } else {
      int n_sel = p.sel_count[r];
      int sl = p.sel_len[r];
      sl = sl < 0 ? 0 : (sl > p.max_ctx ? p.max_ctx : sl);
      n_sel = n_sel < 0 ? 0 : (n_sel > p.sel_stride ? p.sel_stride : n_sel);
      n_sel = n_sel > sl ? sl : n_sel;
      cd[e] = hkv * draft_splits(draft_set_size(n_sel, sl, L));
    }
  }
  {
    int bv = block_excl_scan(cv[0] + cv[1] + cv[2] + cv[3], tmp, &tot);
    if (threadIdx.x == 0) s_misc[0] = tot;
    int bd = block_excl_scan(cd[0] + cd[1] + cd[2] + cd[3], tmp, &tot);
    if (threadIdx.x == 0) s_misc[1] = tot;
    int bs = block_excl_scan(cs[0] + cs[1] + cs[2] + cs[3], tmp, &tot);
    if (threadIdx.x == 0) s_misc[2] = tot;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 4 * threadIdx.x + e;
      if (r < B) {
        s_pv[r] = bv;
        s_pd[r] = bd;
        s_ps[r] = bs;
      }
      bv += cv[e];
      bd += cd[e];
      bs += cs[e];
    }
  }
  __syncthreads();
  const int Tv = s_misc[0], Td = s_misc[1], Ts = s_misc[2];
  const int total = Tv + Td + Ts;

  float* dump_all = reinterpret_cast<float*>(p.ws + wl.dump);
  float* scores_all = reinterpret_cast<float*>(p.ws + wl.scores);
  float* vparts_all = reinterpret_cast<float*>(p.ws + wl.vparts);
  float* dparts_all = reinterpret_cast<float*>(p.ws + wl.dparts);
  uint32_t* vcount = reinterpret_cast<uint32_t*>(p.ws + wl.vcount);
  uint32_t* scount = reinterpret_cast<uint32_t*>(p.ws + wl.scount);
  uint32_t* ready = reinterpret_cast<uint32_t*>(p.ws + wl.ready);
  uint32_t* dcount = reinterpret_cast<uint32_t*>(p.ws + wl.dcount);

  for (;;) {
    __syncthreads();
    if (threadIdx.x == 0) s_misc[8] = (int)atomic_add_agent(&hdr->queue_head, 1u);
    __syncthreads();
    const int t = s_misc[8];
    if (t >= total) break;

    if (t < Tv) {
      // ---------------- verify chunk
      const int r = find_owner(s_pv, B, t);
      const int L = p.ctx_lens[r];
      const int ns = verify_splits(L);
      const int local = t - s_pv[r];
      const int h = local / ns, split = local - (local / ns) * ns;
      const int v = s_vslot[r];
      const int qoff = s_qoff[r];
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
      it.q = p.q + (int64_t)qoff * p.hq * kD;
      it.q_row_stride = (int64_t)p.hq * kD;
      it.dump = dump_all + (int64_t)v * p.hq * kp1 * wl.lstride;
      it.lstride = wl.lstride;
      it.out = p.out + (int64_t)qoff * p.hq * kD;
      it.out_row_stride = (int64_t)p.hq * kD;
      it.lse = p.lse + (int64_t)qoff * p.hq;
      it.lse_row_stride = p.hq;
      it.err = err;
      uint32_t* rdy = ready + (int64_t)v * hkv + h;
      if (ns == 1) {
        verify_chunk<NQT>(it, h, 0, nullptr, lds);
        drain_stores_and_barrier();
        if (threadIdx.x == 0) {
          __threadfence();
          atomic_store_agent(rdy, 1u);
        }
      } else {
        float* parts = vparts_all + ((int64_t)v * hkv + h) * wl.vsplits * M * kPartStride;
        verify_chunk<NQT>(it, h, split, parts + (int64_t)split * M * kPartStride, lds);
        uint32_t* cnt = vcount + (int64_t)v * hkv + h;
        if (arrive_last(cnt, (uint32_t)ns, &flag)) {
          if (threadIdx.x == 0) atomic_store_agent(cnt, 0u);
          verify_combine(it, h, parts, ns);
          drain_stores_and_barrier();
          if (threadIdx.x == 0) {
            __threadfence();
            atomic_store_agent(rdy, 1u);
          }
        }
      }
    } else if (t < Tv + Td) {
      // ---------------- draft chunk
      const int td = t - Tv;
      const int r = find_owner(s_pd, B, td);
      const int qoff = s_qoff[r];
      DraftItem it;
      make_draft_item<G>(it, p.kv, r, p.ctx_lens[r], p.max_ctx, p.sel_idx, p.sel_stride, p.sel_count,
                         p.sel_len, p.q + (int64_t)qoff * p.hq * kD, p.out + (int64_t)qoff * p.hq * kD,
                         p.lse + (int64_t)qoff * p.hq, p.scale, p.hq, err, false);
      const int N = draft_set_size(it.n_sel, it.sel_len, it.L);
      const int ns = draft_splits(N);
      const int local = td - s_pd[r];
      const int h = local / ns, split = local - (local / ns) * ns;
      const int p0 = split * kDraftChunk, p1 = min(p0 + kDraftChunk, N);
      if (ns == 1) {
        draft_range<G>(it, h, 0, N, nullptr, lds);
      } else {
        float* parts = dparts_all + ((int64_t)r * hkv + h) * wl.dsplits * G * kPartStride;
        draft_range<G>(it, h, p0, p1, parts + (int64_t)split * G * kPartStride, lds);
        uint32_t* cnt = dcount + (int64_t)r * hkv + h;
        if (arrive_last(cnt, (uint32_t)ns, &flag)) {
          if (threadIdx.x == 0) atomic_store_agent(cnt, 0u);
          draft_combine<G>(it, h, parts, ns);
        }
      }
    } else {
      // ---------------- score chunk (+ selection by the last one)
      const int ts = t - Tv - Td;
      const int r = find_owner(s_ps, B, ts);
      const int L = p.ctx_lens[r];
      const int ns = score_splits(L);
      const int local = ts - s_ps[r];
      const int h = local / ns, c = local - (local / ns) * ns;
      const int v = s_vslot[r];
      const int qoff = s_qoff[r];
      uint32_t* rdy = ready + (int64_t)v * hkv + h;
      if (threadIdx.x == 0) {
        uint32_t spins = 0;
        while (atomic_load_agent(rdy) == 0u) {
          // bounded: give up (and flag it) after kSpinLimit polls, or at once
          // if another wait of this launch already gave up
          if (++spins > kSpinLimit || (atomic_load_agent(err) & SSPEC_DEV_ERR_WAIT_TIMEOUT)) {
            set_error(err, SSPEC_DEV_ERR_WAIT_TIMEOUT);
            break;
          }
          __builtin_amdgcn_s_sleep(2);
        }
        __threadfence();
      }
      __syncthreads();
      ScoreItem it;
      it.dump = dump_all + (int64_t)v * p.hq * kp1 * wl.lstride;
      it.lstride = wl.lstride;
      it.lse = p.lse + (int64_t)qoff * p.hq;
      it.lse_row_stride = p.hq;
      it.hq = p.hq;
      it.kp1 = kp1;
      it.G = G;
      it.M = M;
      it.L = L;
      it.scores = scores_all + (int64_t)v * hkv * wl.lstride;
      it.sstride = wl.lstride;
      score_chunk(it, h, c, reinterpret_cast<float*>(lds));
      uint32_t* cnt = scount + (int64_t)v * hkv + h;
      if (arrive_last(cnt, (uint32_t)ns, &flag)) {
        if (threadIdx.x == 0) {
          atomic_store_agent(cnt, 0u);
          atomic_store_agent(rdy, 0u);
        }
        const int K = select_count(L, p.s);
        select_topk(it.scores + (int64_t)h * it.sstride, L, K,
                    p.sel_idx + ((int64_t)r * hkv + h) * p.sel_stride, reinterpret_cast<float*>(lds));
        if (threadIdx.x == 0 && h == 0) {
          p.sel_count[r] = K;
          p.sel_len[r] = L;
        }
      }
    }
  }

  // ---- exit: the last work-group out resets the queue for the next launch
  if (threadIdx.x == 0) {
    __threadfence();
    const uint32_t old = atomic_add_agent(&hdr->exit_count, 1u);
    if (old + 1u == gridDim.x) {
      atomic_store_agent(&hdr->queue_head, 0u);
      atomic_store_agent(&hdr->exit_count, 0u);
    }
  }
}

// ------------------------------------------------------------ host side ---
thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(SSPEC_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  return SSPEC_OK;
}

int check_heads(int hq, int hkv, int k) {
  if (hkv < 1 || hq < 1) return fail(SSPEC_ERR_INVALID_ARG, "num_q_heads and num_kv_heads must be >= 1 (got %d, %d)", hq, hkv);
  if (hq % hkv != 0) return fail(SSPEC_ERR_UNSUPPORTED, "num_q_heads (%d) must be a multiple of num_kv_heads (%d)", hq, hkv);
  const int G = hq / hkv;
  if (G > kMaxG) return fail(SSPEC_ERR_UNSUPPORTED, "GQA group size %d > %d", G, kMaxG);
  if (k < 0 || k > kMaxK) return fail(SSPEC_ERR_UNSUPPORTED, "k must be in [0, %d] (got %d)", kMaxK, k);
  if (G * (k + 1) > kMaxRows) return fail(SSPEC_ERR_UNSUPPORTED, "G*(k+1) = %d > %d", G * (k + 1), kMaxRows);
  return SSPEC_OK;
}

int check_kv(const sspec_paged_kv* kv) {
  if (!kv) return fail(SSPEC_ERR_INVALID_ARG, "kv is NULL");
  if (!kv->k_pages || !kv->v_pages || !kv->block_table) return fail(SSPEC_ERR_INVALID_ARG, "kv has a NULL pointer");
  if (kv->head_dim != kD) return fail(SSPEC_ERR_UNSUPPORTED, "head_dim must be %d (got %d)", kD, kv->head_dim);
  if (kv->page_size != kPage) return fail(SSPEC_ERR_UNSUPPORTED, "page_size must be %d (got %d)", kPage, kv->page_size);
  if (kv->num_pages < 1 || kv->bt_stride < 1 || kv->num_seqs < 1 || kv->num_kv_heads < 1)
    return fail(SSPEC_ERR_INVALID_ARG, "kv sizes must be >= 1 (num_pages %d, bt_stride %d, num_seqs %d, num_kv_heads %d)",
                kv->num_pages, kv->bt_stride, kv->num_seqs, kv->num_kv_heads);
  return SSPEC_OK;
}

int check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (!ws) return fail(SSPEC_ERR_WORKSPACE, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(ws) % 256 != 0) return fail(SSPEC_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (ws_bytes < need) return fail(SSPEC_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", ws_bytes, need);
  return SSPEC_OK;
}

// ---- template dispatch tables
template <int NQT>
int launch_verify(const VerifyParams& p, int grid, hipStream_t st) {
  hipLaunchKernelGGL(verify_kernel<NQT>, dim3(grid), dim3(kThreads), 0, st, p);
  return check_launch("verify_kernel");
}
using VerifyFn = int (*)(const VerifyParams&, int, hipStream_t);
template <int NQT>
constexpr VerifyFn verify_entry() {
  if constexpr (SSPEC_ONLY_NQT == 0 || SSPEC_ONLY_NQT == NQT) return &launch_verify<NQT>;
  else return nullptr;
}
const VerifyFn kVerifyFns[8] = {verify_entry<1>(), verify_entry<2>(), verify_entry<3>(), verify_entry<4>(),
                                verify_entry<5>(), verify_entry<6>(), verify_entry<7>(), verify_entry<8>()};

template <int G>
int launch_draft(const DraftParams& p, int grid, hipStream_t st) {
  hipLaunchKernelGGL(draft_kernel<G>, dim3(grid), dim3(kThreads), 0, st, p);
  return check_launch("draft_kernel");
}
using DraftFn = int (*)(const DraftParams&, int, hipStream_t);
template <int G>
constexpr DraftFn draft_entry() {
  if constexpr (SSPEC_ONLY_G == 0 || SSPEC_ONLY_G == G) return &launch_draft<G>;
  else return nullptr;
}
const DraftFn kDraftFns[8] = {draft_entry<1>(), draft_entry<2>(), draft_entry<3>(), draft_entry<4>(),
                              draft_entry<5>(), draft_entry<6>(), draft_entry<7>(), draft_entry<8>()};

std::mutex g_occ_mu;
std::unordered_map<uint64_t, int> g_grid_cache;

template <int G, int NQT>
int launch_unified(const UnifiedParams& p, hipStream_t st) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(SSPEC_ERR_HIP, "hipGetDevice failed");
  const uint64_t key = ((uint64_t)dev << 32) | (uint64_t)(G * 16 + NQT);
  int grid = 0;
  {
    std::lock_guard<std::mutex> lk(g_occ_mu);
    auto f = g_grid_cache.find(key);
    if (f != g_grid_cache.end()) grid = f->second;
  }
  if (grid == 0) {
    int cus = 0, occ = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return fail(SSPEC_ERR_HIP, "hipDeviceGetAttribute failed");
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, unified_kernel<G, NQT>, kThreads, 0) != hipSuccess)
      return fail(SSPEC_ERR_HIP, "hipOccupancyMaxActiveBlocksPerMultiprocessor failed");
    grid = cus * (occ > 0 ? occ : 1);
    std::lock_guard<std::mutex> lk(g_occ_mu);
    g_grid_cache[key] = grid;
  }
  hipLaunchKernelGGL((unified_kernel<G, NQT>), dim3(grid), dim3(kThreads), 0, st, p);
  return check_launch("unified_kernel");
}
using UnifiedFn = int (*)(const UnifiedParams&, hipStream_t);

template <int G, int NQT>
constexpr UnifiedFn unified_entry() {
  if constexpr (NQT <= (G * (kMaxK + 1) + 15) / 16 && NQT <= kMaxRows / 16 &&
                (SSPEC_ONLY_G == 0 || SSPEC_ONLY_G == G) && (SSPEC_ONLY_NQT == 0 || SSPEC_ONLY_NQT == NQT))
    return &launch_unified<G, NQT>;
  else return nullptr;
}
template <int G>
constexpr std::array<UnifiedFn, 8> unified_row() {
  return {unified_entry<G, 1>(), unified_entry<G, 2>(), unified_entry<G, 3>(), unified_entry<G, 4>(),
          unified_entry<G, 5>(), unified_entry<G, 6>(), unified_entry<G, 7>(), unified_entry<G, 8>()};
}
const std::array<UnifiedFn, 8> kUnifiedFns[8] = {unified_row<1>(), unified_row<2>(), unified_row<3>(), unified_row<4>(),
                                                 unified_row<5>(), unified_row<6>(), unified_row<7>(), unified_row<8>()};

}  // namespace

// ==================================================================== ABI ===
extern "C" {

const char* sspec_last_error(void) { return g_last_error.c_str(); }

int sspec_workspace_init(void* ws, size_t ws_bytes, void* stream) {
  if (!ws) return fail(SSPEC_ERR_WORKSPACE, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(ws) % 256 != 0) return fail(SSPEC_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (ws_bytes < sizeof(WsHeader)) return fail(SSPEC_ERR_WORKSPACE, "workspace smaller than its %zu-byte header", sizeof(WsHeader));
  const size_t n = ws_bytes / 4;
  const int grid = (int)std::min<size_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(zero_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, (uint32_t*)ws, n);
  return check_launch("zero_kernel");
}

int sspec_read_device_error(void* ws, int clear, void* stream, uint32_t* flags) {
  if (!ws || !flags) return fail(SSPEC_ERR_INVALID_ARG, "ws and flags must not be NULL");
  hipStream_t st = (hipStream_t)stream;
  if (hipStreamSynchronize(st) != hipSuccess) return fail(SSPEC_ERR_HIP, "hipStreamSynchronize failed");
  uint32_t v = 0;
  if (hipMemcpy(&v, ws, sizeof(v), hipMemcpyDeviceToHost) != hipSuccess) return fail(SSPEC_ERR_HIP, "hipMemcpy failed");
  *flags = v;
  if (clear) {
    const uint32_t z = 0;
    if (hipMemcpy(ws, &z, sizeof(z), hipMemcpyHostToDevice) != hipSuccess) return fail(SSPEC_ERR_HIP, "hipMemcpy failed");
  }
  return SSPEC_OK;
}

size_t sspec_verify_workspace_size(int32_t n, int32_t max_ctx, int32_t num_q_heads, int32_t num_kv_heads, int32_t k) {
  if (n < 0 || max_ctx < 1 || num_kv_heads < 1 || num_q_heads < num_kv_heads || k < 0) return 0;
  return VerifyWs(n, max_ctx, num_q_heads, num_kv_heads, k).total;
}

int sspec_verify_attn(const sspec_paged_kv* kv, const uint16_t* q, const int32_t* seq_ids, const int32_t* ctx_lens,
                      int32_t n, int32_t max_ctx, int32_t num_q_heads, int32_t k, float sm_scale, uint16_t* out,
                      float* lse, float* logits, int64_t logit_stride, void* ws, size_t ws_bytes, void* stream) {
  int rc;
  if ((rc = check_kv(kv))) return rc;
  if ((rc = check_heads(num_q_heads, kv->num_kv_heads, k))) return rc;
  if (n < 0) return fail(SSPEC_ERR_INVALID_ARG, "n must be >= 0 (got %d)", n);
  if (max_ctx < 1) return fail(SSPEC_ERR_INVALID_ARG, "max_ctx must be >= 1 (got %d)", max_ctx);
  if (!std::isfinite(sm_scale)) return fail(SSPEC_ERR_INVALID_ARG, "sm_scale must be finite");
  if (n == 0) return SSPEC_OK;
  if (!q || !seq_ids || !ctx_lens || !out || !lse || !logits) return fail(SSPEC_ERR_INVALID_ARG, "a verify array pointer is NULL");
  if (logit_stride < round_up(max_ctx, kPage) || logit_stride % 4 != 0)
    return fail(SSPEC_ERR_INVALID_ARG, "logit_stride (%lld) must be a multiple of 4 and >= round_up(max_ctx, 16) = %d",
                (long long)logit_stride, round_up(max_ctx, kPage));
  const VerifyWs wl(n, max_ctx, num_q_heads, kv->num_kv_heads, k);
  if ((rc = check_ws(ws, ws_bytes, wl.total))) return rc;
  const int G = num_q_heads / kv->num_kv_heads;
  const int nqt = cdiv(G * (k + 1), 16);
  if (!kVerifyFns[nqt - 1]) return fail(SSPEC_ERR_UNSUPPORTED, "verify kernel for %d query tiles not built", nqt);
  VerifyParams p{*kv, q, seq_ids, ctx_lens, n, max_ctx, num_q_heads, k, sm_scale, out, lse, logits, logit_stride,
                 (uint8_t*)ws, verify_splits(max_ctx)};
  const int64_t grid = (int64_t)n * kv->num_kv_heads * p.vsplit_max;
  if (grid > 0x7fffffff) return fail(SSPEC_ERR_UNSUPPORTED, "grid too large");
  return kVerifyFns[nqt - 1](p, (int)grid, (hipStream_t)stream);
}

size_t sspec_pillar_topk_workspace_size(int32_t n, int32_t max_ctx, int32_t num_kv_heads) {
  if (n < 0 || max_ctx < 1 || num_kv_heads < 1) return 0;
  return TopkWs(n, max_ctx, num_kv_heads).total;
}

int sspec_pillar_topk(const float* logits, const float* lse, int64_t logit_stride, const int32_t* seq_ids,
                      const int32_t* ctx_lens, int32_t n, int32_t num_seqs, int32_t max_ctx, int32_t num_q_heads,
                      int32_t num_kv_heads, int32_t k, double s, int32_t* sel_idx, int32_t sel_stride,
                      int32_t* sel_count, int32_t* sel_len, void* ws, size_t ws_bytes, void* stream) {
  int rc;
  if ((rc = check_heads(num_q_heads, num_kv_heads, k))) return rc;
  if (n < 0 || num_seqs < 1 || max_ctx < 1)
    return fail(SSPEC_ERR_INVALID_ARG, "bad sizes (n %d, num_seqs %d, max_ctx %d)", n, num_seqs, max_ctx);
  if (!(s > 0.0 && s <= 1.0)) return fail(SSPEC_ERR_INVALID_ARG, "s must be in (0, 1] (got %g)", s);
  if (n == 0) return SSPEC_OK;
  if (!logits || !lse || !seq_ids || !ctx_lens || !sel_idx || !sel_count || !sel_len)
    return fail(SSPEC_ERR_INVALID_ARG, "a pillar_topk array pointer is NULL");
  if (logit_stride < round_up(max_ctx, kPage) || logit_stride % 4 != 0)
    return fail(SSPEC_ERR_INVALID_ARG, "logit_stride (%lld) must be a multiple of 4 and >= round_up(max_ctx, 16)",
                (long long)logit_stride);
  if (sel_stride < select_count(max_ctx, s))
    return fail(SSPEC_ERR_INVALID_ARG, "sel_stride (%d) < ceil(s*max_ctx) = %d", sel_stride, select_count(max_ctx, s));
  const TopkWs wl(n, max_ctx, num_kv_heads);
  if ((rc = check_ws(ws, ws_bytes, wl.total))) return rc;
  TopkParams p{logits, lse, logit_stride, seq_ids, ctx_lens, n, num_seqs, max_ctx, num_q_heads, num_kv_heads, k, s,
               sel_idx, sel_stride, sel_count, sel_len, (uint8_t*)ws, score_splits(max_ctx)};
  const int64_t grid = (int64_t)n * num_kv_heads * p.ssplit_max;
  if (grid > 0x7fffffff) return fail(SSPEC_ERR_UNSUPPORTED, "grid too large");
  hipLaunchKernelGGL(topk_kernel, dim3((int)grid), dim3(kThreads), 0, (hipStream_t)stream, p);
  return check_launch("topk_kernel");
}

size_t sspec_draft_workspace_size(int32_t n, int32_t num_q_heads, int32_t num_kv_heads) {
  if (n < 0 || num_kv_heads < 1 || num_q_heads < num_kv_heads) return 0;
  return DraftWs(n, num_q_heads, num_kv_heads).total;
}

int sspec_sparse_draft_attn(const sspec_paged_kv* kv, const uint16_t* q, const int32_t* seq_ids, const int32_t* ctx_lens,
                            const int32_t* sel_idx, int32_t sel_stride, const int32_t* sel_count, const int32_t* sel_len,
                            int32_t n, int32_t max_ctx, int32_t num_q_heads, float sm_scale, uint16_t* out, float* lse,
                            void* ws, size_t ws_bytes, void* stream) {
  int rc;
  if ((rc = check_kv(kv))) return rc;
  if ((rc = check_heads(num_q_heads, kv->num_kv_heads, 0))) return rc;
  if (n < 0 || max_ctx < 1 || sel_stride < 0)
    return fail(SSPEC_ERR_INVALID_ARG, "bad sizes (n %d, max_ctx %d, sel_stride %d)", n, max_ctx, sel_stride);
  if (!std::isfinite(sm_scale)) return fail(SSPEC_ERR_INVALID_ARG, "sm_scale must be finite");
  if (n == 0) return SSPEC_OK;
  if (!q || !seq_ids || !ctx_lens || !sel_count || !sel_len || !out || (!sel_idx && sel_stride > 0))
    return fail(SSPEC_ERR_INVALID_ARG, "a draft array pointer is NULL");
  const DraftWs wl(n, num_q_heads, kv->num_kv_heads);
  if ((rc = check_ws(ws, ws_bytes, wl.total))) return rc;
  DraftParams p{*kv, q, seq_ids, ctx_lens, sel_idx, sel_stride, sel_count, sel_len, n, max_ctx, num_q_heads, sm_scale,
                out, lse, (uint8_t*)ws};
  const int64_t grid = (int64_t)n * kv->num_kv_heads;
  if (grid > 0x7fffffff) return fail(SSPEC_ERR_UNSUPPORTED, "grid too large");
  const int G = num_q_heads / kv->num_kv_heads;
  if (!kDraftFns[G - 1]) return fail(SSPEC_ERR_UNSUPPORTED, "draft kernel for G=%d not built", G);
  return kDraftFns[G - 1](p, (int)grid, (hipStream_t)stream);
}

size_t sspec_unified_workspace_size(int32_t num_seqs, int32_t max_verify, int32_t max_ctx, int32_t num_q_heads,
                                    int32_t num_kv_heads, int32_t k) {
  if (num_seqs < 1 || max_verify < 0 || max_ctx < 1 || num_kv_heads < 1 || num_q_heads < num_kv_heads || k < 0) return 0;
  return UnifiedWs(num_seqs, max_verify, max_ctx, num_q_heads, num_kv_heads, k).total;
}

int sspec_unified_attn(const sspec_paged_kv* kv, const uint16_t* q, const int32_t* ctx_lens, const int32_t* bucket_ids,
                       int32_t verify_bucket, int32_t num_seqs, int32_t max_verify, int32_t max_ctx, int32_t num_q_heads,
                       int32_t k, double s, float sm_scale, int32_t* sel_idx, int32_t sel_stride, int32_t* sel_count,
                       int32_t* sel_len, uint16_t* out, float* lse, void* ws, size_t ws_bytes, void* stream) {
  int rc;
  if ((rc = check_kv(kv))) return rc;
  if ((rc = check_heads(num_q_heads, kv->num_kv_heads, k))) return rc;
  if (num_seqs < 1 || num_seqs > kMaxSeqsUnified)
    return fail(SSPEC_ERR_UNSUPPORTED, "num_seqs must be in [1, %d] (got %d)", kMaxSeqsUnified, num_seqs);
  if (num_seqs > kv->num_seqs) return fail(SSPEC_ERR_INVALID_ARG, "num_seqs (%d) > kv->num_seqs (%d)", num_seqs, kv->num_seqs);
  if (max_verify < 0 || max_ctx < 1) return fail(SSPEC_ERR_INVALID_ARG, "bad sizes (max_verify %d, max_ctx %d)", max_verify, max_ctx);
  if (!(s > 0.0 && s <= 1.0)) return fail(SSPEC_ERR_INVALID_ARG, "s must be in (0, 1] (got %g)", s);
  if (!std::isfinite(sm_scale)) return fail(SSPEC_ERR_INVALID_ARG, "sm_scale must be finite");
  if (!q || !ctx_lens || !bucket_ids || !sel_idx || !sel_count || !sel_len || !out || !lse)
    return fail(SSPEC_ERR_INVALID_ARG, "a unified array pointer is NULL");
  if (sel_stride < select_count(max_ctx, s))
    return fail(SSPEC_ERR_INVALID_ARG, "sel_stride (%d) < ceil(s*max_ctx) = %d", sel_stride, select_count(max_ctx, s));
  const UnifiedWs wl(num_seqs, max_verify, max_ctx, num_q_heads, kv->num_kv_heads, k);
  if ((rc = check_ws(ws, ws_bytes, wl.total))) return rc;
  const int G = num_q_heads / kv->num_kv_heads;
  const int nqt = cdiv(G * (k + 1), 16);
  UnifiedFn fn = kUnifiedFns[G - 1][nqt - 1];
  if (!fn) return fail(SSPEC_ERR_UNSUPPORTED, "no unified kernel for G=%d, %d query tiles", G, nqt);
  UnifiedParams p{*kv, q, ctx_lens, bucket_ids, verify_bucket, num_seqs, max_verify, max_ctx, num_q_heads, k, s,
                  sm_scale, sel_idx, sel_stride, sel_count, sel_len, out, lse, (uint8_t*)ws};
  return fn(p, (hipStream_t)stream);
}

}  // extern "C"

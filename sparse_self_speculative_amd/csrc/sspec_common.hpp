// Shared device helpers, work geometry and workspace layout of the SparseSpec
// attention path on gfx950 (CDNA4: wave64, 16x16 bf16 MFMA, 160 KB LDS/CU).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sspec.h"

namespace sspec {

constexpr int kD = 128;        // head_dim
constexpr int kPage = 16;      // tokens per page
constexpr int kWave = 64;
constexpr int kThreads = 256;  // 4 waves per work-group
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxG = 8;
constexpr int kMaxK = 16;
constexpr int kMaxRows = 128;  // G*(k+1)
constexpr int kMaxSeqsUnified = 1024;
constexpr int kMaxCtx = 1 << 20;   // longest supported context (tokens)

// Work geometry.  A verify task covers a page-aligned chunk of keys of one
// (request, KV head); a score task a chunk of dumped logits; a draft task a
// chunk of the draft token set.  Host and device use the same functions.
constexpr int kVerifyChunk = 1024;
constexpr int kVerifySplitCap = 64;
constexpr int kScoreChunk = 1024;
constexpr int kDraftChunk = 2048;     // set positions per unified draft task
constexpr int kDraftSub = 2048;       // positions whose row ids sit in LDS at once

__host__ __device__ inline int cdiv(int a, int b) { return (a + b - 1) / b; }
__host__ __device__ inline int64_t cdiv64(int64_t a, int64_t b) { return (a + b - 1) / b; }
__host__ __device__ inline int round_up(int a, int b) { return cdiv(a, b) * b; }

__host__ __device__ inline int verify_chunk_len(int L) {
  int c = round_up(cdiv(L, kVerifySplitCap), kPage);
  return c > kVerifyChunk ? c : kVerifyChunk;
}
__host__ __device__ inline int verify_splits(int L) { return L <= 0 ? 0 : cdiv(L, verify_chunk_len(L)); }
__host__ __device__ inline int score_splits(int L) { return L <= 0 ? 0 : cdiv(L, kScoreChunk); }
__host__ __device__ inline int draft_splits(int N) { return N <= 0 ? 1 : cdiv(N, kDraftChunk); }
// A draft set holds at most max(L, sel_len) <= max_ctx positions once the
// selected count is clamped to sel_len (valid selections are distinct
// indices below sel_len), so draft_splits(max_ctx) bounds every request.

// Selection count K = min(L, ceil(s*L)), s*L in IEEE double.
__host__ __device__ inline int select_count(int L, double s) {
  double x = ceil(s * (double)L);
  return x >= (double)L ? L : (int)x;
}

// Rows of a verify partial: m, l, o[128].
constexpr int kPartStride = kD + 2;

// ------------------------------------------------------------------ bf16 ---
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ uint32_t f2bf_bits(float f) {
  // round to nearest even; NaN stays a quiet NaN
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  return f2bf_bits(lo) | (f2bf_bits(hi) << 16);
}
// Split two fp32 values into bf16 high parts (packed) and bf16 low parts
// (the rounded remainders, packed); hi + lo equals the fp32 value to about
// 2^-17 relative, where one bf16 alone leaves 2^-9.
__device__ __forceinline__ void split_bf2(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  const uint32_t h0 = f2bf_bits(x0), h1 = f2bf_bits(x1);
  hi = h0 | (h1 << 16);
  lo = pack_bf2(x0 - __uint_as_float(h0 << 16), x1 - __uint_as_float(h1 << 16));
}

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t v) { return __builtin_bit_cast(bf16x2, v); }

// 16x16x32 bf16 MFMA: D = A(16x32) * B(32x16) + C.  A lane l holds row l%16,
// B lane l holds column l%16, both with the same 8 k-slots per lane; the
// f32 result has lane l holding column l%16, rows 4*(l/16)+r in reg r.
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t sel_half(uint32_t lo_src, uint32_t hi_src, int odd) {
  // pack element (odd ? high : low) half of lo_src into bits 0..15 and the
  // same half of hi_src into bits 16..31
  return odd ? __builtin_amdgcn_perm(hi_src, lo_src, 0x07060302u)
             : __builtin_amdgcn_perm(hi_src, lo_src, 0x05040100u);
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a), as_bf16x2(b), c, false);
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();
// Online softmax keeps a reference max per row and only moves it when the
// running max exceeds it by more than this (natural-log units), so
// un-normalised probabilities stay <= e^8 and rescales are rare.
constexpr float kRescale = 8.f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

typedef __attribute__((ext_vector_type(4))) short s16x4;
// 16x16x16 bf16 MFMA (4 k-slots per lane), same row/column/result layout.
__device__ __forceinline__ f32x4 mfma16x16x16(uint32_t a0, uint32_t a1, uint32_t b0, uint32_t b1, f32x4 c) {
  typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
  const s16x4 a = __builtin_bit_cast(s16x4, u32x2{a0, a1});
  const s16x4 b = __builtin_bit_cast(s16x4, u32x2{b0, b1});
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// ------------------------------------------------------- cross-lane ops ---
#define SSPEC_DPP(x, ctrl) __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), ctrl, 0xF, 0xF, false))
// sum over the 16 lanes of each DPP row (every lane gets the row sum)
__device__ __forceinline__ float row16_sum(float x) {
  x += SSPEC_DPP(x, 0xB1);   // quad_perm [1,0,3,2]
  x += SSPEC_DPP(x, 0x4E);   // quad_perm [2,3,0,1]
  x += SSPEC_DPP(x, 0x141);  // row_half_mirror
  x += SSPEC_DPP(x, 0x140);  // row_mirror
  return x;
}
// partner values 16 and 32 lanes away (v_permlane16/32_swap on gfx950):
// with both operands x, the two results are x of the lane pair, in some order
__device__ __forceinline__ float max_xor16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ------------------------------------------------------------ atomics ----
__device__ __forceinline__ void set_error(uint32_t* err, uint32_t bit) {
  __hip_atomic_fetch_or(err, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t atomic_add_agent(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t atomic_load_agent(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void atomic_store_agent(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Every wave waits until its own global stores are acknowledged, then the
// work-group meets at a barrier.  A plain barrier does not wait for other
// waves' stores; after this one, an agent-scope release by any one thread
// (which writes back this XCD's L2) covers the stores of the whole group.
__device__ __forceinline__ void drain_stores_and_barrier() {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), expcnt/lgkmcnt untouched
  __syncthreads();
}

// Work-group "last one out" test: every work-group that finished one part of
// a job calls this after its global writes; exactly one (the last) gets true
// and then sees all the other parts' writes.  The counter is reset to 0 by
// the caller that got true, so the workspace stays reusable.
__device__ __forceinline__ bool arrive_last(uint32_t* counter, uint32_t expected, int* lds_flag) {
  drain_stores_and_barrier();
  if (threadIdx.x == 0) {
    __threadfence();
    uint32_t old = atomic_add_agent(counter, 1u);
    bool last = (old + 1u == expected);
    if (last) __threadfence();
    *lds_flag = last ? 1 : 0;
  }
  __syncthreads();
  return *lds_flag != 0;
}

// ----------------------------------------------------- workspace header ---
struct WsHeader {
  uint32_t err;
  uint32_t queue_head;
  uint32_t exit_count;
  uint32_t pad[61];
};
static_assert(sizeof(WsHeader) == 256, "workspace header must be 256 bytes");

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Workspace carve-up of each entry point: host computes sizes from the
// arguments, device recomputes the same offsets.
struct VerifyWs {
  size_t counters, parts, total;
  __host__ __device__ VerifyWs(int n, int max_ctx, int hq, int hkv, int k) {
    const int M = (hq / hkv) * (k + 1);
    const int ns = verify_splits(max_ctx);
    counters = align256(sizeof(WsHeader));
    parts = counters + align256(sizeof(uint32_t) * (size_t)n * hkv);
    total = parts + align256(sizeof(float) * (size_t)n * hkv * ns * M * kPartStride);
  }
};

struct TopkWs {
  size_t counters, scores, total;
  int lstride;
  __host__ __device__ TopkWs(int n, int max_ctx, int hkv) {
    lstride = round_up(max_ctx > 0 ? max_ctx : 1, kPage);
    counters = align256(sizeof(WsHeader));
    scores = counters + align256(sizeof(uint32_t) * (size_t)n * hkv);
    total = scores + align256(sizeof(float) * (size_t)n * hkv * lstride);
  }
};

struct DraftWs {
  size_t total;
  __host__ __device__ DraftWs(int, int, int) { total = align256(sizeof(WsHeader)); }
};

struct UnifiedWs {
  size_t vcount, scount, ready, dcount, dump, scores, vparts, dparts, total;
  int lstride;   // dump / score row stride (floats)
  int vsplits;   // verify splits per (verify item, KV head), upper bound
  int dsplits;   // draft splits per (request, KV head), upper bound
  __host__ __device__ UnifiedWs(int num_seqs, int max_verify, int max_ctx, int hq, int hkv, int k) {
    const int G = hq / hkv, M = G * (k + 1);
    lstride = round_up(max_ctx > 0 ? max_ctx : 1, kPage);
    vsplits = verify_splits(max_ctx);
    dsplits = draft_splits(max_ctx);
    const size_t nvh = (size_t)max_verify * hkv;
    vcount = align256(sizeof(WsHeader));
    scount = vcount + align256(sizeof(uint32_t) * nvh);
    ready = scount + align256(sizeof(uint32_t) * nvh);
    dcount = ready + align256(sizeof(uint32_t) * nvh);
    dump = dcount + align256(sizeof(uint32_t) * (size_t)num_seqs * hkv);
    scores = dump + align256(sizeof(float) * (size_t)max_verify * hq * (k + 1) * lstride);
    vparts = scores + align256(sizeof(float) * nvh * lstride);
    dparts = vparts + align256(sizeof(float) * nvh * vsplits * M * kPartStride);
    total = dparts + align256(sizeof(float) * (size_t)num_seqs * hkv * dsplits * G * kPartStride);
  }
};

}  // namespace sspec

// Shared device helpers, work geometry and workspace layout of the SparseSpec
// attention path on gfx950 (CDNA4: wave64, 16x16 bf16 MFMA, 160 KB LDS/CU).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "sspec.h"

// Task bodies (one per wave task) are compiled as calls or inlined.
// (inlined: a call would turn the LDS pointers into flat pointers, whose
// accesses count against vmcnt and break the explicit-wait pipelines)
#ifndef SSPEC_TASK
#define SSPEC_TASK __forceinline__
#endif

namespace sspec {

constexpr int kD = 128;        // head_dim
constexpr int kPage = 16;      // tokens per page
constexpr int kWave = 64;
constexpr int kMaxG = 8;
constexpr int kMaxK = 16;
constexpr int kMaxRows = 128;  // G*(k+1)
constexpr int kMaxItems = 512;     // requests per launch of any entry point
constexpr int kMaxCtx = 1 << 20;   // longest supported context (tokens)

// Work geometry.  A verify task covers a page-aligned chunk of keys of one
// (request, KV head); a score task a chunk of dumped logits; a draft task a
// chunk of the draft token set.  Host and device use the same functions.
#ifndef SSPEC_VCHUNK_MIN
#define SSPEC_VCHUNK_MIN 64
#endif
constexpr int kVChunkMin = SSPEC_VCHUNK_MIN;        // pages per verify task, fewest (1024 keys)
constexpr int kVChunkMax = 256;       // pages per verify task, most (4096 keys)
#ifndef SSPEC_SCORE_CHUNK
#define SSPEC_SCORE_CHUNK 2048
#endif
constexpr int kScoreChunk = SSPEC_SCORE_CHUNK;     // keys per score task of a unified launch (one wave);
                                                   // also the unit of the score rows and selection bitmaps
#ifndef SSPEC_SCORE_CHUNK_SEL
#define SSPEC_SCORE_CHUNK_SEL 1024
#endif
// keys per score task of a selection-only launch: it runs nothing else, so
// shorter tasks on more waves finish its score phase sooner
constexpr int kScoreChunkSel = SSPEC_SCORE_CHUNK_SEL;
static_assert(kScoreChunk % kScoreChunkSel == 0 && kScoreChunkSel % 256 == 0, "score chunk lengths");
#ifndef SSPEC_DRAFT_CHUNK
#define SSPEC_DRAFT_CHUNK 512
#endif
constexpr int kDraftChunk = SSPEC_DRAFT_CHUNK;      // set positions per draft task (one wave), at most
constexpr int kDraftSub = 512;        // positions whose row ids sit in LDS at once
constexpr int kHistBins = 2048;       // bins of the selection's 11-bit radix digit

__host__ __device__ constexpr int cdiv(int a, int b) { return (a + b - 1) / b; }
__host__ __device__ inline int64_t cdiv64(int64_t a, int64_t b) { return (a + b - 1) / b; }
__host__ __device__ inline int round_up(int a, int b) { return cdiv(a, b) * b; }
// ceil(a / b) for 0 <= a < 2^24, 0 < b <= 2^8, by a float quotient corrected
// to the exact integer one (far fewer instructions than integer division)
__device__ __forceinline__ int cdiv_small(int a, int b) {
  int q = (int)((float)a / (float)b);
  q -= q * b > a;
  q += (q + 1) * b <= a;
  return q + (q * b < a);
}

// Verify chunks of a context of L keys at cp pages per chunk.
__host__ __device__ inline int verify_splits(int L, int cp) { return L <= 0 ? 0 : cdiv(cdiv(L, kPage), cp); }
// Pages per verify chunk for one launch: a launch whose verify pages (all
// (request, KV head) pairs together: `pages`, over `pairs` pairs) can be cut
// into at most one chunk per worker wave gets the shortest chunks that do
// it, so every verify starts at once and none waits for a second round;
// otherwise chunks are kVChunkMin pages and the queue balances them.  With
// the ceiling below, sum over pairs of ceil(p/cp) <= pages/cp + pairs <= workers.
__host__ __device__ inline int verify_chunk_pages(int64_t pages, int pairs, int workers) {
  if (pairs <= 0 || workers <= pairs) return kVChunkMin;
  const int64_t cp = cdiv64(pages, (int64_t)(workers - pairs));
  if (cp > kVChunkMax) return kVChunkMin;
  return cp < kVChunkMin ? kVChunkMin : (int)cp;
}
// Chunk pages of one pair of context L (lmax: longest verify context of the
// launch, 0: no shortening).  A pair's selection starts only after all its
// chunks, and a longer context takes longer to score and select; its chunks
// are shortened by cp * f/256 with f = 104*L/lmax, up to 41% (never below
// kVChunkMin), so that its verify ends earlier.  Shortening the longest by
// half made the medium contexts' full-length chunks end last, and their
// score and selection chains then set the end of the launch.
#ifndef SSPEC_VSHORT
#define SSPEC_VSHORT 104
#endif
__host__ __device__ inline int verify_pair_frac(int L, int lmax) { return lmax > 0 ? (SSPEC_VSHORT * L) / lmax : 0; }
__host__ __device__ inline int verify_pair_chunk_f(int cp, int f) {
  const int c = cp - ((cp * f) >> 8);
  return c < kVChunkMin ? kVChunkMin : c;
}
__host__ __device__ inline int verify_pair_chunk(int cp, int L, int lmax) {
  return verify_pair_chunk_f(cp, verify_pair_frac(L, lmax));
}
__host__ __device__ inline int score_splits(int L, int chunk = kScoreChunk) { return L <= 0 ? 0 : cdiv(L, chunk); }
__host__ __device__ inline int draft_splits(int N) { return N <= 0 ? 1 : cdiv(N, kDraftChunk); }
// Naive batching: a draft is cut like a verify, into chunks of the launch's
// verify chunk length (cp pages of positions; never shorter than
// kDraftChunk, so draft_splits bounds these splits too).
__host__ __device__ inline int naive_draft_splits(int N, int cp) {
  const int c = cp * kPage > kDraftChunk ? cp * kPage : kDraftChunk;
  return N <= 0 ? 1 : cdiv(N, c);
}
// A draft set holds at most max(L, sel_len) <= max_ctx positions once the
// selected count is clamped to sel_len (valid selections are distinct
// indices below sel_len), so draft_splits(max_ctx) bounds every request.

// Selection count K = min(L, ceil(s*L)), s*L in IEEE double.
__host__ __device__ inline int select_count(int L, double s) {
  double x = ceil(s * (double)L);
  return x >= (double)L ? L : (int)x;
}

// Split partial of `rows` attention rows (a verify or draft chunk): the O
// rows [rows][128 floats], then (m, l, 0, 0) per row; the split's size is a
// multiple of 64 bytes.  Within a 512-byte O row the 16-byte units are kept
// in the order the MFMA accumulators hold them, unit 4*j + grp (j = 2r + nh)
// holding dims 32*grp + 8*r + 4*nh .. +3: the four lane groups of an
// accumulator column then write one whole 64-byte segment per store
// instruction (scattered 16-byte pieces, written through to memory by the
// coherent stores, each cost a partial-line write request).
__host__ __device__ constexpr uint32_t part_split_bytes(int rows) {
  return ((uint32_t)rows * (kD + 4) * 4u + 63u) & ~63u;
}
__host__ __device__ constexpr uint32_t part_split_floats(int rows) { return part_split_bytes(rows) / 4u; }
// 16-byte unit of a partial O row that holds dims d .. d+3 (d % 4 == 0)
__host__ __device__ constexpr int part_unit(int d) { return (((d >> 2) & 7) << 2) | (d >> 5); }

// ------------------------------------------------------------------ bf16 ---
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
// Two fp32 values to packed bf16 (round to nearest even): one
// v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf2_t;
  const bf2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
// Split two fp32 values into bf16 high parts (packed) and bf16 low parts
// (the rounded remainders, packed); hi + lo equals the fp32 value to about
// 2^-17 relative, where one bf16 alone leaves 2^-9.
__device__ __forceinline__ void split_bf2(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  hi = pack_bf2(x0, x1);
  lo = pack_bf2(x0 - bf_lo(hi), x1 - bf_hi(hi));
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
// Verify keeps one softmax reference per column for a whole pass over its
// chunk and restarts the pass when the logits climb more than this above it
// (natural-log units: exp(64) ~ 6e27 leaves fp32 and bf16 ample headroom).
constexpr float kVerifyRange = 64.f;

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

// ------------------------------------------- cross-work-group protocol ---
// Data one work-group writes for another (chunk partials, the logit dump,
// LSE, scores) goes through device-coherent accesses: stores and loads with
// the sc1 bit, which is what agent-scope relaxed atomics lower to on this
// GPU.  A writer drains its stores (s_waitcnt vmcnt(0): they have reached
// the coherence point) before it bumps a counter or sets a flag with a
// relaxed atomic; a reader that has seen the counter or flag then reads with
// sc1 loads.  No L2 write-back or invalidate (buffer_wbl2 / buffer_inv) is
// ever needed, which an agent-scope fence would issue on every use.
// Buffer resource over [base, base + bytes) (base wave-uniform): loads past
// the end return 0.  With the sc1 cache-policy bit the loads are
// device-coherent, and the compiler still tracks them like any load.
constexpr int kSc1 = 16;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ f32x4 ld_coh4(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, kSc1));
}
__device__ __forceinline__ u32x4 ld_coh4u(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, kSc1));
}
// o *= alpha on an MFMA accumulator in place: the "a" constraints keep it in
// AGPRs, where the MFMAs want it (a plain multiply made the compiler copy
// every accumulator to VGPRs and back around the loop that holds it); the
// trailing wait states cover an MFMA that reads the registers next.
__device__ __forceinline__ void scale_acc(f32x4& o, float alpha) {
  float t;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float e = o[i];
    asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1\n\ts_nop 4"
                 : "+a"(e), "=&v"(t)
                 : "v"(alpha));
    o[i] = e;
  }
}

// Device-coherent 16-byte store through a buffer resource: an offset past
// the resource's size writes nothing, so a lane can opt out without a branch.
__device__ __forceinline__ void st_coh4_buf(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, (int)byte_off, 0, kSc1);
}
__device__ __forceinline__ void st_coh2u_buf(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, uint32_t a, uint32_t b) {
  typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;
  __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{a, b}, r, (int)byte_off, 0, kSc1);
}
__device__ __forceinline__ float ld_coh1(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)byte_off, 0, kSc1));
}
// The lane index, through an opaque move: every task body derives its
// per-lane addresses from it, and the opaque value keeps the compiler from
// hoisting those out of the persistent loop, where the hoisted values of all
// task kinds would stay live together and exhaust the register file.
__device__ __forceinline__ uint32_t lane_id() {
  uint32_t l = threadIdx.x & 63;
  asm volatile("" : "+v"(l));
  return l;
}
// number of set bits of a wave ballot below this lane
__device__ __forceinline__ uint32_t lanemask_lt_count(uint64_t b) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0u));
}
// The same pointer for the whole wave, in scalar registers.
template <class T>
__device__ __forceinline__ T* wave_uniform(T* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<T*>((uintptr_t)(((uint64_t)hi << 32) | lo));
}
__device__ __forceinline__ void drain_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void st_coh4(float* p, f32x4 v) {
  // a store of more than 8 bytes needs 1 wait state before its data
  // registers may be overwritten
  asm volatile("global_store_dwordx4 %0, %1, off sc1\n\ts_nop 0" ::"v"(p), "v"(v) : "memory");
}
__device__ __forceinline__ void st_coh(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_coh(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_coh_u(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coh_u(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wave "last one out": every wave that finished one part of a job calls
// this after its coherent stores; exactly one (the last) gets true and may
// then read the other parts with coherent loads.  The caller that got true
// resets the counter, so the workspace stays reusable.
__device__ __forceinline__ bool wave_arrive_last(uint32_t* counter, uint32_t expected) {
  drain_vm();
  uint32_t old = 0;
  if (lane_id() == 0) old = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  old = __builtin_amdgcn_readfirstlane(old);
  return old + 1u == expected;
}
// Publish a flag after this wave's coherent stores.
__device__ __forceinline__ void wave_publish(uint32_t* flag, uint32_t v) {
  drain_vm();
  if (lane_id() == 0) st_coh_u(flag, v);
}

// Integer wave reductions and scans on DPP (every lane of the wave active).
// update_dpp with old = 0: a lane whose DPP source lies outside its 16-lane
// row reads 0.
#define SSPEC_DPP_I(x, ctrl) __builtin_amdgcn_update_dpp(0, (x), (ctrl), 0xF, 0xF, false)

// Exclusive prefix sum over the 64 lanes of a wave; *total gets the sum.
// Inclusive prefix within each 16-lane row (row shifts by 1, 2, 4, 8), then
// the totals of the rows before, read from their last lanes.
__device__ __forceinline__ int wave_excl_scan(int v, int* total) {
  const int lane = (int)lane_id();
  int x = v;
  x += SSPEC_DPP_I(x, 0x111);   // row_shr:1
  x += SSPEC_DPP_I(x, 0x112);   // row_shr:2
  x += SSPEC_DPP_I(x, 0x114);   // row_shr:4
  x += SSPEC_DPP_I(x, 0x118);   // row_shr:8
  const int r0 = __builtin_amdgcn_readlane(x, 15);
  const int r1 = __builtin_amdgcn_readlane(x, 31);
  const int r2 = __builtin_amdgcn_readlane(x, 47);
  const int r3 = __builtin_amdgcn_readlane(x, 63);
  const int row = lane >> 4;
  x += (row > 0 ? r0 : 0) + (row > 1 ? r1 : 0) + (row > 2 ? r2 : 0);
  *total = r0 + r1 + r2 + r3;
  return x - v;
}
// Sum / maximum over the 64 lanes of a wave (every lane gets it): within
// each row by quad permutes and mirrors, then over the four rows.
__device__ __forceinline__ int wave_sum_i(int x) {
  x += SSPEC_DPP_I(x, 0xB1);    // quad_perm [1,0,3,2]
  x += SSPEC_DPP_I(x, 0x4E);    // quad_perm [2,3,0,1]
  x += SSPEC_DPP_I(x, 0x141);   // row_half_mirror
  x += SSPEC_DPP_I(x, 0x140);   // row_mirror
  return __builtin_amdgcn_readlane(x, 0) + __builtin_amdgcn_readlane(x, 16) + __builtin_amdgcn_readlane(x, 32) +
         __builtin_amdgcn_readlane(x, 48);
}
__device__ __forceinline__ int wave_max_i(int x) {
  x = max(x, SSPEC_DPP_I(x, 0xB1));
  x = max(x, SSPEC_DPP_I(x, 0x4E));
  x = max(x, SSPEC_DPP_I(x, 0x141));
  x = max(x, SSPEC_DPP_I(x, 0x140));
  return max(max(__builtin_amdgcn_readlane(x, 0), __builtin_amdgcn_readlane(x, 16)),
             max(__builtin_amdgcn_readlane(x, 32), __builtin_amdgcn_readlane(x, 48)));
}

// ----------------------------------------------------- workspace header ---
// The counters that many waves touch sit on separate 128-byte lines.
// The launch-wide counters are split into kShards independent copies, one
// per XCD (work-group b runs on XCD b % 8): an atomic on one address costs
// about 12 ns at the memory side, so 1024 waves claiming work at the same
// moment would queue for ~12 us on a single counter.
constexpr int kShards = 8;
struct WsHeader {
  struct alignas(128) Ctr {
    uint32_t queue_head;   // static tasks handed out from this shard
    uint32_t exit_count;   // waves of this shard that have left the launch
    uint32_t pad[30];
  };
  struct alignas(128) Sq {
    uint64_t sq;           // published score tasks of this shard's list: low half
                           // = next to hand out, high half = published so far
    uint32_t pad[30];
  };
  uint32_t err;            // SSPEC_DEV_ERR_* bits
  uint32_t trace_count;    // task-trace records written (trace builds)
  uint32_t trace_off;      // byte offset / 256 of the trace records (trace builds)
  uint32_t exit_shards;    // shards whose waves have all left
  uint32_t magic;          // kWsMagic once sspec_workspace_init has cleared the workspace
  uint32_t aborted;        // set by a wave that gave up a bounded wait in this launch
  uint64_t clean_end;      // bytes [kZoneBegin, clean_end) of the workspace are zero (see WsLayout)
  uint32_t sel_path[4];    // selections run, by Top-K path (bitmaps, threshold-bin collection, two
                           // global passes; [3] unused) -- diagnostic, never reset by a launch
  uint32_t pad0[20];
  Ctr ctr[kShards];
  Sq sq[kShards];
  __host__ __device__ uint32_t* sq_head(int x) { return reinterpret_cast<uint32_t*>(&sq[x].sq); }
  __host__ __device__ uint32_t* sq_reserve(int x) { return reinterpret_cast<uint32_t*>(&sq[x].sq) + 1; }
};
static_assert(sizeof(WsHeader) == 128 * (1 + 2 * kShards), "workspace header layout");
static_assert(offsetof(WsHeader, clean_end) == 24 && offsetof(WsHeader, sel_path) == 32, "header fields");
constexpr uint32_t kWsMagic = 0x53535043u;   // "SSPC"

__host__ __device__ constexpr size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
constexpr size_t kZoneBegin = align256(sizeof(WsHeader));

// Task trace (compile with -DSSPEC_TRACE=1): one record per task, times from
// the 100 MHz constant clock.  Development builds only.
#ifndef SSPEC_TRACE
#define SSPEC_TRACE 0
#endif
struct TraceRec {
  uint64_t t0, t1;
  uint32_t kind_worker;   // kind | worker << 8
  uint32_t item, h, chunk;
};
constexpr size_t kTraceRecords = SSPEC_TRACE ? (size_t)1 << 20 : 0;
enum TraceKind : uint32_t {
  kTrVerify = 1, kTrVCombine = 2, kTrScore = 3, kTrSelect = 4, kTrDraft = 5, kTrDCombine = 6, kTrIdle = 7,
  kTrPrologue = 8, kTrCollect = 12, kTrSelPrep = 13, kTrArrive = 14
};
constexpr int kTrPhases = 9;   // prologue phase stamps of a trace build

// Entries of the published score-task list sit 128 bytes apart (each is
// polled by the one wave that owns it).
constexpr int kSlistStride = 32;

// What one launch of the persistent kernel does.
enum Mode : int { kModeVerify = 0, kModeTopk = 1, kModeDraft = 2, kModeUnified = 3 };

// Workspace carve-up, the same on host and device.  n = items of one launch
// (requests in unified mode; a call over more than kMaxItems items uses the
// layout of kMaxItems for every launch), nv = verify slots, ns = score slots.
//
// Zero-state zone.  The regions [kZoneBegin, zone_end) -- the arrival
// counters, the published score-task list and the Top-K histograms -- must
// read zero when a launch starts, and every launch that completes leaves
// them zero again (whoever consumes a counter, an entry or a histogram
// resets it).  Every layout starts its zone at kZoneBegin; the data regions
// (dump, scores, partials) follow the zone, so a call with another layout
// may leave data where this layout keeps zero state.  The header's
// clean_end records how far the zero prefix reaches: the host clears
// [kZoneBegin, zone_end) before a launch whose zone_end passes it, and the
// kernel refuses to run (SSPEC_DEV_ERR_WS_STATE) if it still does.
struct WsLayout {
  size_t vcount, scount, dcount, slist, ghist, dump, scores, tops, selbits, vparts, dparts, trace, total;
  size_t zone_end;   // = dump: end of the zero-state zone
  int64_t lstride;   // keys per KV head in the dump (unified)
  int64_t sstride;   // score row stride (floats)
  int vsplits;       // key chunks per verify (item, KV head), upper bound
  int dsplits;       // set chunks per draft (item, KV head), upper bound
  int nslist;        // entries of the published score-task list
  __host__ __device__ __attribute__((always_inline)) WsLayout(int mode, int n, int max_verify, int max_ctx, int hq,
                                                              int hkv, int k) {
    const int G = hq / hkv, M = G * (k + 1);
    const int mc = max_ctx > 0 ? max_ctx : 1;
    const bool uni = mode == kModeUnified;
    const size_t nv = mode == kModeVerify ? n : (uni ? max_verify : 0);
    const size_t ns = mode == kModeTopk ? n : (uni ? max_verify : 0);
    const size_t nd = (mode == kModeDraft || uni) ? n : 0;
    lstride = round_up(mc, kPage);
    sstride = round_up(mc, kScoreChunk);
    vsplits = verify_splits(mc, kVChunkMin);
    dsplits = draft_splits(mc);
    nslist = uni ? (int)(nv * hkv * score_splits(mc)) : 0;
    vcount = kZoneBegin;
    scount = vcount + align256(sizeof(uint32_t) * nv * hkv);
    dcount = scount + align256(sizeof(uint32_t) * ns * hkv);
    slist = dcount + align256(sizeof(uint32_t) * nd * hkv);
    ghist = slist + align256(sizeof(uint32_t) * kSlistStride * (size_t)nslist);
    dump = ghist + align256(sizeof(uint32_t) * ns * hkv * kHistBins);
    zone_end = dump;
    scores = dump + align256(uni ? sizeof(float) * nv * hkv * (size_t)lstride * round_up(M, 4) : 0);
    // the scores' top 16 bits, read by the classification pass
    tops = scores + align256(sizeof(float) * ns * hkv * (size_t)sstride);
    selbits = tops + align256(sizeof(uint16_t) * ns * hkv * (size_t)sstride);
    // per pair, the selection's two bitmaps per score chunk
    vparts = selbits + align256(sizeof(uint32_t) * ns * hkv * (size_t)(sstride / 16));
    dparts = vparts + align256(vsplits > 1 ? (size_t)part_split_bytes(M) * nv * hkv * vsplits : 0);
    trace = dparts + align256(dsplits > 1 ? (size_t)part_split_bytes(G) * nd * hkv * dsplits : 0);
    total = trace + align256(kTraceRecords * sizeof(TraceRec));
  }
};

}  // namespace sspec

// Paged KV cache maintenance around the attention of one iteration [talk
// notes "Accelerating Large-Scale Reasoning Model Inference with Sparse
// Self-Speculative Decoding", sections Dynamic KV-Cache management (paper
// §4.4: every decode step adds the new tokens' KV) and Delayed verification
// (paper §4.3: the verify decides which drafts are accepted)]:
//
//   sspec_kv_append    writes the current tokens' key/value rows into their
//                      pages (k+1 rows for a verifying request, 1 for a
//                      drafting one), before the attention reads them;
//   sspec_kv_rollback  after a verify, cuts a request's context back to the
//                      accepted tokens and its selection length with it.
//
// Both are pure data movement / integer work: one 16-byte load and store per
// lane, rows of 256 bytes (one KV head of one token) copied whole.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdint>

#include "sspec.h"

namespace sspec {

int fail(int code, const char* fmt, ...);
int check_launch(const char* what);

namespace {

constexpr int kD = 128;
constexpr int kPage = 16;
constexpr int kAppendThreads = 256;

// Block (r, i): row i of request r (if it has one), every KV head, K and V.
// Thread t copies 16-byte chunk t % 16 of head (t / 16) / 2's K (even) or V
// (odd) row, for heads t/32, t/32 + 8, ...  The request's row offset is the
// number of rows of the requests before it: r + k * (verifying requests
// before r), counted by the block.  The kernel is latency-bound (one
// iteration moves a few MB), so every load that does not depend on another
// is issued first: the request's bucket and context with the counting
// loads, then the new rows together with the block-table entry.
__global__ __launch_bounds__(kAppendThreads) void kv_append_kernel(
    uint16_t* __restrict__ kp, uint16_t* __restrict__ vp, const int32_t* __restrict__ bt, int num_pages,
    int hkv, int bt_stride, const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    const int32_t* __restrict__ ctx_lens, const int32_t* __restrict__ bucket_ids, int verify_bucket, int k,
    const int32_t* __restrict__ seq_ids, int num_slots, uint32_t* err) {
  const int r = blockIdx.x, i = blockIdx.y, tid = threadIdx.x;
  // item r's request slot: its context length and block-table row
  const int q = seq_ids ? seq_ids[r] : r;
  if (q < 0 || q >= num_slots) {
    if (i == 0 && tid == 0 && err) atomicOr(err, SSPEC_DEV_ERR_SEQ_RANGE);
    return;
  }
  const int b = bucket_ids[r], c = ctx_lens[q];
  __shared__ int s_cnt[kAppendThreads / 64];
  int cnt = 0;
  for (int j = tid; j < r; j += kAppendThreads) cnt += bucket_ids[j] == verify_bucket;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) cnt += __shfl_xor(cnt, off);
  if ((tid & 63) == 0) s_cnt[tid >> 6] = cnt;
  __syncthreads();
  const int n = b == verify_bucket ? k + 1 : 1;
  if (i >= n) return;
  int vbefore = 0;
#pragma unroll
  for (int w = 0; w < kAppendThreads / 64; ++w) vbefore += s_cnt[w];
  const int64_t row = (int64_t)r + (int64_t)k * vbefore + i;
  const int pos = c - n + i;
  if (pos < 0 || (int64_t)pos >= (int64_t)bt_stride * kPage) {
    if (tid == 0 && err) atomicOr(err, SSPEC_DEV_ERR_CTX_RANGE);
    return;
  }
  const int chunk = tid & 15, kv = (tid >> 4) & 1;
  const uint16_t* src = kv ? v_new : k_new;
  uint16_t* dst = kv ? vp : kp;
  const int h0 = tid >> 5;
  uint4 x0 = {0, 0, 0, 0};
  if (h0 < hkv) x0 = *reinterpret_cast<const uint4*>(src + (row * hkv + h0) * kD + chunk * 8);
  const int page = bt[(int64_t)q * bt_stride + pos / kPage];
  if (page < 0 || page >= num_pages) {
    if (tid == 0 && err) atomicOr(err, SSPEC_DEV_ERR_PAGE_RANGE);
    return;
  }
  uint16_t* prow = dst + ((int64_t)page * hkv * kPage + pos % kPage) * kD + chunk * 8;
  if (h0 < hkv) *reinterpret_cast<uint4*>(prow + (int64_t)h0 * kPage * kD) = x0;
  for (int h = h0 + kAppendThreads / 32; h < hkv; h += kAppendThreads / 32) {
    const uint4 x = *reinterpret_cast<const uint4*>(src + (row * hkv + h) * kD + chunk * 8);
    *reinterpret_cast<uint4*>(prow + (int64_t)h * kPage * kD) = x;
  }
}

__global__ void kv_rollback_kernel(const int32_t* __restrict__ bucket_ids, int verify_bucket,
                                   const int32_t* __restrict__ accepted, int num_seqs, int k, int32_t* ctx_lens,
                                   int32_t* sel_len) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= num_seqs || bucket_ids[r] != verify_bucket) return;
  const int a = min(max(accepted[r], 0), k);
  const int c = ctx_lens[r] - (k - a);
  ctx_lens[r] = c;
  sel_len[r] = min(sel_len[r], c);
}

}  // namespace
}  // namespace sspec

using namespace sspec;

namespace sspec {
int kv_append_impl(const sspec_paged_kv* kv, const uint16_t* k_new, const uint16_t* v_new, const int32_t* ctx_lens,
                   const int32_t* bucket_ids, int32_t verify_bucket, int32_t num_seqs, int32_t k, const int32_t* seq_ids,
                   uint32_t* err, void* stream) {
  if (!kv) return fail(SSPEC_ERR_INVALID_ARG, "kv is NULL");
  if (!kv->k_pages || !kv->v_pages || !kv->block_table) return fail(SSPEC_ERR_INVALID_ARG, "kv has a NULL pointer");
  if (kv->head_dim != kD) return fail(SSPEC_ERR_UNSUPPORTED, "head_dim must be %d (got %d)", kD, kv->head_dim);
  if (kv->page_size != kPage) return fail(SSPEC_ERR_UNSUPPORTED, "page_size must be %d (got %d)", kPage, kv->page_size);
  if (kv->num_pages < 1 || kv->bt_stride < 1 || kv->num_seqs < 1 || kv->num_kv_heads < 1)
    return fail(SSPEC_ERR_INVALID_ARG, "kv sizes must be >= 1");
  if (k < 0 || k > 16) return fail(SSPEC_ERR_UNSUPPORTED, "k must be in [0, 16] (got %d)", k);
  if (num_seqs < 0 || num_seqs > kv->num_seqs)
    return fail(SSPEC_ERR_INVALID_ARG, "num_seqs (%d) must be in [0, kv->num_seqs = %d]", num_seqs, kv->num_seqs);
  if (num_seqs == 0) return SSPEC_OK;
  if (!k_new || !v_new || !ctx_lens || !bucket_ids) return fail(SSPEC_ERR_INVALID_ARG, "a kv_append array pointer is NULL");
  if ((reinterpret_cast<uintptr_t>(k_new) | reinterpret_cast<uintptr_t>(v_new) |
       reinterpret_cast<uintptr_t>(kv->k_pages) | reinterpret_cast<uintptr_t>(kv->v_pages)) % 16 != 0)
    return fail(SSPEC_ERR_INVALID_ARG, "k_new, v_new and the pools must be 16-byte aligned");
  hipLaunchKernelGGL(kv_append_kernel, dim3(num_seqs, k + 1), dim3(kAppendThreads), 0, (hipStream_t)stream,
                     const_cast<uint16_t*>(kv->k_pages), const_cast<uint16_t*>(kv->v_pages), kv->block_table,
                     kv->num_pages, kv->num_kv_heads, kv->bt_stride, k_new, v_new, ctx_lens, bucket_ids,
                     verify_bucket, k, seq_ids, kv->num_seqs, err);
  return check_launch("kv_append_kernel");
}
}  // namespace sspec

extern "C" {

int sspec_kv_append(const sspec_paged_kv* kv, const uint16_t* k_new, const uint16_t* v_new, const int32_t* ctx_lens,
                    const int32_t* bucket_ids, int32_t verify_bucket, int32_t num_seqs, int32_t k, uint32_t* err,
                    void* stream) {
  return kv_append_impl(kv, k_new, v_new, ctx_lens, bucket_ids, verify_bucket, num_seqs, k, nullptr, err, stream);
}

int sspec_kv_append_slots(const sspec_paged_kv* kv, const uint16_t* k_new, const uint16_t* v_new,
                          const int32_t* seq_ids, const int32_t* ctx_lens, const int32_t* bucket_ids,
                          int32_t verify_bucket, int32_t num_items, int32_t k, uint32_t* err, void* stream) {
  if (!seq_ids) return fail(SSPEC_ERR_INVALID_ARG, "seq_ids is NULL");
  return kv_append_impl(kv, k_new, v_new, ctx_lens, bucket_ids, verify_bucket, num_items, k, seq_ids, err, stream);
}

int sspec_kv_rollback(const int32_t* bucket_ids, int32_t verify_bucket, const int32_t* accepted, int32_t num_seqs,
                      int32_t k, int32_t* ctx_lens, int32_t* sel_len, void* stream) {
  if (k < 0 || k > 16) return fail(SSPEC_ERR_UNSUPPORTED, "k must be in [0, 16] (got %d)", k);
  if (num_seqs < 0) return fail(SSPEC_ERR_INVALID_ARG, "num_seqs must be >= 0 (got %d)", num_seqs);
  if (num_seqs == 0) return SSPEC_OK;
  if (!bucket_ids || !accepted || !ctx_lens || !sel_len)
    return fail(SSPEC_ERR_INVALID_ARG, "a kv_rollback array pointer is NULL");
  hipLaunchKernelGGL(kv_rollback_kernel, dim3((num_seqs + 255) / 256), dim3(256), 0, (hipStream_t)stream, bucket_ids,
                     verify_bucket, accepted, num_seqs, k, ctx_lens, sel_len);
  return check_launch("kv_rollback_kernel");
}

}  // extern "C"

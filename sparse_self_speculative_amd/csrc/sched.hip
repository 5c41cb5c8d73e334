// The unified batch scheduler with delayed verification [talk notes
// "Accelerating Large-Scale Reasoning Model Inference with Sparse
// Self-Speculative Decoding", sections Unified batch scheduler (paper §4.2,
// Fig. 8: requests are spread over k+1 buckets, a new request joining the
// least-loaded one; each iteration runs k draft buckets and one verify
// bucket) and Delayed verification (paper §4.3, Fig. 9: the host consumes an
// iteration's verify results one iteration later, so it never waits for the
// GPU inside an iteration; only the verifying requests wait, for one
// iteration)].
//
// Host-side state only.  Every request owns a stable slot (the row of its
// block table, context length and selection state on the device); each
// iteration's batch lists the slots that run, in admission order, with
// their buckets, and the host's copy of every slot's context length and
// selection length.  Token accounting per request (the attention kernels'
// conventions): every iteration it runs appends one position (a draft adds
// a draft token; a verify adds the last draft and checks the drafts made
// since the previous verify); a verify of a request holding d drafts that
// accepts a of them cuts the context by d - a and commits a + 1 tokens.
//
// sspec_accept_stub stands in for the model's acceptance test: request q's
// verify in iteration t accepts the leading drafts j = 0, 1, ... for which a
// counter-based uniform u(q, t, j) (SplitMix64 of the triple) is below the
// acceptance rate, at most k of them.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <deque>
#include <new>
#include <vector>

#include "sspec.h"

namespace sspec {

int fail(int code, const char* fmt, ...);
int check_launch(const char* what);

namespace {

// SplitMix64 finaliser (Steele, Lea, Flood 2014), also used to seed xorshift
// generators: one 64-bit counter in, one well-mixed 64-bit value out.
__host__ __device__ inline uint64_t splitmix64(uint64_t x) {
  x += 0x9E3779B97F4A7C15ull;
  x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
  x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
  return x ^ (x >> 31);
}

__global__ void accept_stub_kernel(const int32_t* __restrict__ req_ids, const int32_t* __restrict__ seq_ids,
                                   const int32_t* __restrict__ bucket_ids, int verify_bucket, int n, int k,
                                   int64_t iter, double rate, uint64_t seed, int num_slots,
                                   int32_t* __restrict__ accepted) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n || bucket_ids[i] != verify_bucket) return;
  const int slot = seq_ids[i];
  if (slot < 0 || slot >= num_slots) return;
  const uint64_t base = seed ^ ((uint64_t)(uint32_t)req_ids[i] << 40) ^ ((uint64_t)iter << 8);
  int a = 0;
  while (a < k) {
    const double u = (double)(splitmix64(base ^ (uint64_t)a) >> 11) * 0x1.0p-53;
    if (!(u < rate)) break;
    ++a;
  }
  accepted[slot] = a;
}

}  // namespace
}  // namespace sspec

using namespace sspec;

struct SchedReq {
  int32_t id = -1;
  int32_t bucket = 0;
  int32_t ctx = 0;        // positions written (the context the next attention sees, minus its new one)
  int32_t sel_len = 0;    // the device's selection length for this slot
  int32_t drafts = 0;     // draft iterations since the last resolved verify
  int32_t out = 0;        // committed output tokens
  int32_t max_new = 0;
  bool live = false;
  bool waiting = false;   // verified; its result is not yet resolved
  int64_t ready = 0;      // first iteration it may run again (a verify at t: t+1, delayed t+2)
};

struct SchedVerify {
  int32_t slot, drafts;
};

struct sspec_sched {
  int32_t k, kp1, max_slots;
  bool delayed;
  int64_t iter = 0;                                             // next iteration to form
  std::vector<int32_t> loads;                                   // live requests per bucket
  std::vector<SchedReq> slots;
  std::vector<int32_t> order;                                   // live slots in admission order
  std::deque<std::pair<int64_t, std::vector<SchedVerify>>> unresolved;   // formed, not yet resolved
};

extern "C" {

int sspec_sched_create(int32_t k, int32_t max_slots, int32_t delayed, sspec_sched** out) {
  if (!out) return fail(SSPEC_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (k < 0 || k > 16) return fail(SSPEC_ERR_UNSUPPORTED, "k must be in [0, 16] (got %d)", k);
  if (max_slots < 1 || max_slots > (1 << 20)) return fail(SSPEC_ERR_INVALID_ARG, "max_slots must be in [1, 2^20]");
  sspec_sched* s = new (std::nothrow) sspec_sched();
  if (!s) return fail(SSPEC_ERR_INVALID_ARG, "out of host memory");
  s->k = k;
  s->kp1 = k + 1;
  s->max_slots = max_slots;
  s->delayed = delayed != 0;
  s->loads.assign(k + 1, 0);
  s->slots.resize(max_slots);
  *out = s;
  return SSPEC_OK;
}

int sspec_sched_destroy(sspec_sched* s) {
  delete s;
  return SSPEC_OK;
}

int sspec_sched_admit(sspec_sched* s, int32_t req_id, int32_t prompt_len, int32_t max_new, int32_t* slot,
                      int32_t* bucket) {
  if (!s) return fail(SSPEC_ERR_INVALID_ARG, "scheduler is NULL");
  if (req_id < 0 || prompt_len < 0 || max_new < 1)
    return fail(SSPEC_ERR_INVALID_ARG, "req_id >= 0, prompt_len >= 0 and max_new >= 1 are required");
  int free_slot = -1;
  for (int32_t i = 0; i < s->max_slots; ++i) {
    if (s->slots[i].live && s->slots[i].id == req_id)
      return fail(SSPEC_ERR_INVALID_ARG, "request %d is already admitted", req_id);
    if (!s->slots[i].live && free_slot < 0) free_slot = i;
  }
  if (free_slot < 0) return fail(SSPEC_ERR_WORKSPACE, "no free slot (max_slots = %d)", s->max_slots);
  // greedy bin packing: the bucket with the fewest live requests, lowest id on ties
  int32_t b = 0;
  for (int32_t x = 1; x < s->kp1; ++x)
    if (s->loads[x] < s->loads[b]) b = x;
  SchedReq& r = s->slots[free_slot];
  r = SchedReq();
  r.id = req_id;
  r.bucket = b;
  r.ctx = prompt_len;
  r.max_new = max_new;
  r.live = true;
  ++s->loads[b];
  s->order.push_back(free_slot);
  if (slot) *slot = free_slot;
  if (bucket) *bucket = b;
  return SSPEC_OK;
}

int sspec_sched_next(sspec_sched* s, int32_t* req_ids, int32_t* seq_ids, int32_t* bucket_ids, int32_t* n_items,
                     int32_t* n_verify, int32_t* verify_bucket, int64_t* iter, int32_t* ctx_lens, int32_t* sel_len) {
  if (!s || !seq_ids || !bucket_ids || !n_items || !ctx_lens || !sel_len)
    return fail(SSPEC_ERR_INVALID_ARG, "an output pointer is NULL");
  // the iteration whose results must be resolved before this one is formed
  const int64_t need = s->iter - (s->delayed ? 2 : 1);
  if (!s->unresolved.empty() && s->unresolved.front().first <= need)
    return fail(SSPEC_ERR_INVALID_ARG, "resolve iteration %lld before forming iteration %lld",
                (long long)s->unresolved.front().first, (long long)s->iter);
  const int32_t vb = (int32_t)(s->iter % s->kp1);
  int32_t n = 0, nv = 0;
  std::vector<SchedVerify> vers;
  for (int32_t slot : s->order) {
    SchedReq& r = s->slots[slot];
    if (r.waiting || s->iter < r.ready) continue;
    r.ctx += 1;
    if (r.bucket == vb) {
      vers.push_back({slot, r.drafts});
      r.waiting = true;
      r.ready = s->iter + (s->delayed ? 2 : 1);
      r.sel_len = r.ctx;   // the verify rewrites the slot's selection over its whole context
      ++nv;
    } else {
      r.drafts += 1;
    }
    if (req_ids) req_ids[n] = r.id;
    seq_ids[n] = slot;
    bucket_ids[n] = r.bucket;
    ++n;
  }
  for (int32_t i = 0; i < s->max_slots; ++i) {
    const SchedReq& r = s->slots[i];
    ctx_lens[i] = r.live ? r.ctx : 0;
    sel_len[i] = r.live ? r.sel_len : 0;
  }
  *n_items = n;
  if (n_verify) *n_verify = nv;
  if (verify_bucket) *verify_bucket = vb;
  if (iter) *iter = s->iter;
  s->unresolved.push_back({s->iter, std::move(vers)});
  ++s->iter;
  return SSPEC_OK;
}

int sspec_sched_resolve(sspec_sched* s, int64_t iter, const int32_t* accepted_by_slot, int32_t* finished, int32_t cap,
                        int32_t* n_finished) {
  if (!s || !accepted_by_slot || !n_finished) return fail(SSPEC_ERR_INVALID_ARG, "a pointer is NULL");
  if (cap < 0 || (cap > 0 && !finished)) return fail(SSPEC_ERR_INVALID_ARG, "bad finished array");
  if (s->unresolved.empty() || s->unresolved.front().first != iter)
    return fail(SSPEC_ERR_INVALID_ARG, "iteration %lld is not the oldest unresolved one", (long long)iter);
  *n_finished = 0;
  for (const SchedVerify& v : s->unresolved.front().second) {
    SchedReq& r = s->slots[v.slot];
    const int32_t a = std::min(std::max(accepted_by_slot[v.slot], 0), v.drafts);
    r.ctx -= v.drafts - a;
    r.sel_len = std::min(r.sel_len, r.ctx);
    r.out += a + 1;
    r.drafts = 0;
    r.waiting = false;
    if (r.out >= r.max_new) {
      if (*n_finished < cap) finished[*n_finished] = r.id;
      ++*n_finished;
      --s->loads[r.bucket];
      r.live = false;
      s->order.erase(std::find(s->order.begin(), s->order.end(), v.slot));
    }
  }
  s->unresolved.pop_front();
  return SSPEC_OK;
}

int sspec_sched_query(const sspec_sched* s, int32_t slot, int32_t* req_id, int32_t* ctx, int32_t* out_tokens,
                      int32_t* bucket) {
  if (!s || slot < 0 || slot >= s->max_slots) return fail(SSPEC_ERR_INVALID_ARG, "bad scheduler or slot");
  const SchedReq& r = s->slots[slot];
  if (req_id) *req_id = r.live ? r.id : -1;
  if (ctx) *ctx = r.ctx;
  if (out_tokens) *out_tokens = r.out;
  if (bucket) *bucket = r.bucket;
  return SSPEC_OK;
}

int sspec_accept_stub(const int32_t* req_ids, const int32_t* seq_ids, const int32_t* bucket_ids, int32_t verify_bucket,
                      int32_t n_items, int32_t k, int64_t iter, double rate, uint64_t seed, int32_t num_slots,
                      int32_t* accepted_by_slot, void* stream) {
  if (k < 0 || k > 16) return fail(SSPEC_ERR_UNSUPPORTED, "k must be in [0, 16] (got %d)", k);
  if (n_items < 0 || num_slots < 1) return fail(SSPEC_ERR_INVALID_ARG, "n_items >= 0 and num_slots >= 1 required");
  if (!(rate >= 0.0 && rate <= 1.0)) return fail(SSPEC_ERR_INVALID_ARG, "rate must be in [0, 1]");
  if (n_items == 0) return SSPEC_OK;
  if (!req_ids || !seq_ids || !bucket_ids || !accepted_by_slot)
    return fail(SSPEC_ERR_INVALID_ARG, "an array pointer is NULL");
  hipLaunchKernelGGL(accept_stub_kernel, dim3((n_items + 255) / 256), dim3(256), 0, (hipStream_t)stream, req_ids,
                     seq_ids, bucket_ids, verify_bucket, n_items, k, iter, rate, seed, num_slots, accepted_by_slot);
  return check_launch("accept_stub_kernel");
}

}  // extern "C"

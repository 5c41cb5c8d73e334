// Dynamic KV-cache offload [talk notes "Accelerating Large-Scale Reasoning
// Model Inference with Sparse Self-Speculative Decoding", section Dynamic
// KV-Cache management, paper §4.4: the GPU is filled with KV caches of as
// many requests as fit; when it runs short, requests' caches move to host
// memory asynchronously, a chunk at a time, and come back the same way, both
// in FIFO order so that no request waits behind later ones].
//
// Two parts:
//   * data movers (device): sspec_kv_pack_pages gathers whole pages (K and
//     V blocks of every KV head) of a page list into one contiguous buffer,
//     sspec_kv_unpack_pages scatters such a buffer back into a page list.
//     Pure copies, bit for bit;
//   * the offload engine (host): a FIFO of evict / restore jobs, each cut
//     into chunks of at most chunk_pages pages.  sspec_offload_pump issues
//     chunks, in FIFO order, on a side stream given by the caller: an evict
//     chunk is packed into a device staging slot and copied to the job's
//     place in a pinned host arena by the copy engine (no compute units
//     involved in the transfer); a restore chunk is copied from the host
//     arena into a staging slot and unpacked into the job's new pages.
//     Each chunk records an event on the side stream; sspec_offload_poll
//     retires finished chunks without blocking and reports jobs whose last
//     chunk has finished, again in FIFO order.
// The engine allocates no device memory: the caller passes the staging
// buffer and the pinned host arena.  The page ids a chunk's kernel reads sit
// in a small table at the head of the pinned arena (the kernel reads them
// over the host link: a few hundred bytes per chunk).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <deque>
#include <list>
#include <new>
#include <vector>

#include "sspec.h"

namespace sspec {

int fail(int code, const char* fmt, ...);
int check_launch(const char* what);

namespace {

constexpr int kD = 128;
constexpr int kPage = 16;
constexpr int kMoveThreads = 256;

// Block (i, kv): page pages[i]'s K (kv = 0) or V (kv = 1) block, hkv*4 KB,
// to or from buffer block 2*i + kv.  16 bytes per thread per step.
template <bool PACK>
__global__ __launch_bounds__(kMoveThreads) void kv_move_kernel(uint16_t* __restrict__ kp, uint16_t* __restrict__ vp,
                                                               int num_pages, int hkv,
                                                               const int32_t* __restrict__ pages,
                                                               uint16_t* __restrict__ buf, uint32_t* err) {
  const int i = blockIdx.x, kv = blockIdx.y;
  const int page = pages[i];
  if (page < 0 || page >= num_pages) {
    if (threadIdx.x == 0 && err) atomicOr(err, SSPEC_DEV_ERR_PAGE_RANGE);
    return;
  }
  const int64_t block = (int64_t)hkv * kPage * kD;   // bf16 elements of one pool's page
  uint16_t* pool = (kv ? vp : kp) + (int64_t)page * block;
  uint16_t* b = buf + (2 * (int64_t)i + kv) * block;
  const int n16 = (int)(block / 8);                    // 16-byte pieces
  for (int c = threadIdx.x; c < n16; c += kMoveThreads) {
    if (PACK) *reinterpret_cast<uint4*>(b + 8 * c) = *reinterpret_cast<const uint4*>(pool + 8 * c);
    else *reinterpret_cast<uint4*>(pool + 8 * c) = *reinterpret_cast<const uint4*>(b + 8 * c);
  }
}

int check_move_args(const sspec_paged_kv* kv, const int32_t* pages, int32_t n, const void* buf) {
  if (!kv) return fail(SSPEC_ERR_INVALID_ARG, "kv is NULL");
  if (!kv->k_pages || !kv->v_pages) return fail(SSPEC_ERR_INVALID_ARG, "kv has a NULL pool pointer");
  if (kv->head_dim != kD) return fail(SSPEC_ERR_UNSUPPORTED, "head_dim must be %d (got %d)", kD, kv->head_dim);
  if (kv->page_size != kPage) return fail(SSPEC_ERR_UNSUPPORTED, "page_size must be %d (got %d)", kPage, kv->page_size);
  if (kv->num_pages < 1 || kv->num_kv_heads < 1) return fail(SSPEC_ERR_INVALID_ARG, "kv sizes must be >= 1");
  if (n < 0 || n > 65535) return fail(SSPEC_ERR_INVALID_ARG, "n_pages must be in [0, 65535] (got %d)", n);
  if (n == 0) return SSPEC_OK;
  if (!pages || !buf) return fail(SSPEC_ERR_INVALID_ARG, "pages or the buffer is NULL");
  if ((reinterpret_cast<uintptr_t>(buf) | reinterpret_cast<uintptr_t>(kv->k_pages) |
       reinterpret_cast<uintptr_t>(kv->v_pages)) % 16 != 0)
    return fail(SSPEC_ERR_INVALID_ARG, "the buffer and the pools must be 16-byte aligned");
  return SSPEC_OK;
}

int launch_move(bool pack, const sspec_paged_kv* kv, const int32_t* pages, int32_t n, uint16_t* buf, uint32_t* err,
                hipStream_t st) {
  if (pack)
    hipLaunchKernelGGL(kv_move_kernel<true>, dim3(n, 2), dim3(kMoveThreads), 0, st, const_cast<uint16_t*>(kv->k_pages),
                       const_cast<uint16_t*>(kv->v_pages), kv->num_pages, kv->num_kv_heads, pages, buf, err);
  else
    hipLaunchKernelGGL(kv_move_kernel<false>, dim3(n, 2), dim3(kMoveThreads), 0, st,
                       const_cast<uint16_t*>(kv->k_pages), const_cast<uint16_t*>(kv->v_pages), kv->num_pages,
                       kv->num_kv_heads, pages, buf, err);
  return check_launch(pack ? "kv_pack_pages" : "kv_unpack_pages");
}

}  // namespace
}  // namespace sspec

using namespace sspec;

// ------------------------------------------------------------ the engine
struct OffloadJob {
  int32_t req;
  int32_t kind;                  // SSPEC_OFFLOAD_EVICT / SSPEC_OFFLOAD_RESTORE
  std::vector<int32_t> pages;    // device pages read (evict) or written (restore)
  size_t host_page;              // first page of the job's host copy, in page units
  int32_t issued = 0;            // pages issued so far
  int32_t chunks_left = 0;       // chunks issued and not yet retired
};

struct OffloadChunk {
  OffloadJob* job;
  int32_t first, count, slot;
};

struct sspec_offload {
  sspec_paged_kv kv;
  int32_t chunk_pages, slots;
  size_t page_bytes;             // one page's K and V blocks
  uint8_t* staging;              // device: slots * chunk_pages * page_bytes
  uint8_t* host;                 // pinned host arena
  size_t host_pages;             // pages the arena holds after the id table
  int32_t* ids;                  // pinned: [slots][chunk_pages] page ids of the chunk in each slot
  uint8_t* data;                 // pinned: host page copies
  hipStream_t side;
  bool dry;
  std::vector<hipEvent_t> ev;    // one per slot
  std::vector<int32_t> free_slots;
  std::list<OffloadJob> fifo;    // jobs not yet retired, in FIFO order
  std::deque<OffloadChunk> inflight;
  std::vector<std::pair<size_t, size_t>> host_free;   // (first page, pages), sorted, coalesced
  std::vector<int32_t> trace;    // issued chunks: req, kind, first, count (dry-run and tests)
  struct Home {
    int32_t req;
    size_t at;                   // first host page of the request's copy
    int32_t n;                   // pages
  };
  std::vector<Home> homes;       // requests with a host copy (evicted, not yet restored)
};

namespace {

size_t host_alloc(sspec_offload* e, size_t n) {
  for (size_t i = 0; i < e->host_free.size(); ++i) {
    auto& f = e->host_free[i];
    if (f.second >= n) {
      const size_t at = f.first;
      f.first += n;
      f.second -= n;
      if (f.second == 0) e->host_free.erase(e->host_free.begin() + (long)i);
      return at;
    }
  }
  return SIZE_MAX;
}

void host_free(sspec_offload* e, size_t at, size_t n) {
  auto& v = e->host_free;
  auto it = std::lower_bound(v.begin(), v.end(), std::make_pair(at, (size_t)0));
  it = v.insert(it, {at, n});
  // coalesce with the neighbours
  size_t i = (size_t)(it - v.begin());
  if (i + 1 < v.size() && v[i].first + v[i].second == v[i + 1].first) {
    v[i].second += v[i + 1].second;
    v.erase(v.begin() + (long)i + 1);
  }
  if (i > 0 && v[i - 1].first + v[i - 1].second == v[i].first) {
    v[i - 1].second += v[i].second;
    v.erase(v.begin() + (long)i);
  }
}

const sspec_offload::Home* find_home(const sspec_offload* e, int32_t req) {
  for (auto& h : e->homes)
    if (h.req == req) return &h;
  return nullptr;
}

}  // namespace

extern "C" {

int sspec_kv_pack_pages(const sspec_paged_kv* kv, const int32_t* pages, int32_t n_pages, uint16_t* dst, uint32_t* err,
                        void* stream) {
  int rc = check_move_args(kv, pages, n_pages, dst);
  if (rc || n_pages == 0) return rc;
  return launch_move(true, kv, pages, n_pages, dst, err, (hipStream_t)stream);
}

int sspec_kv_unpack_pages(const sspec_paged_kv* kv, const int32_t* pages, int32_t n_pages, const uint16_t* src,
                          uint32_t* err, void* stream) {
  int rc = check_move_args(kv, pages, n_pages, src);
  if (rc || n_pages == 0) return rc;
  return launch_move(false, kv, pages, n_pages, const_cast<uint16_t*>(src), err, (hipStream_t)stream);
}

size_t sspec_offload_page_bytes(int32_t num_kv_heads) {
  return num_kv_heads < 1 ? 0 : (size_t)2 * num_kv_heads * kPage * kD * 2;
}

size_t sspec_offload_host_bytes(int32_t num_kv_heads, int32_t chunk_pages, int32_t slots, int64_t host_pages) {
  if (num_kv_heads < 1 || chunk_pages < 1 || slots < 1 || host_pages < 0) return 0;
  const size_t table = ((size_t)slots * chunk_pages * 4 + 255) / 256 * 256;
  return table + (size_t)host_pages * sspec_offload_page_bytes(num_kv_heads);
}

int sspec_offload_create(const sspec_paged_kv* kv, int32_t chunk_pages, int32_t slots, void* staging,
                         size_t staging_bytes, void* host, size_t host_bytes, void* side_stream, int32_t flags,
                         sspec_offload** out) {
  if (!out) return fail(SSPEC_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  const bool dry = (flags & SSPEC_OFFLOAD_DRY) != 0;
  if (flags & ~SSPEC_OFFLOAD_DRY) return fail(SSPEC_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
  if (!kv) return fail(SSPEC_ERR_INVALID_ARG, "kv is NULL");
  if (kv->head_dim != kD || kv->page_size != kPage)
    return fail(SSPEC_ERR_UNSUPPORTED, "head_dim must be %d and page_size %d", kD, kPage);
  if (kv->num_pages < 1 || kv->num_kv_heads < 1) return fail(SSPEC_ERR_INVALID_ARG, "kv sizes must be >= 1");
  if (!dry && (!kv->k_pages || !kv->v_pages)) return fail(SSPEC_ERR_INVALID_ARG, "kv has a NULL pool pointer");
  if (chunk_pages < 1 || chunk_pages > 4096 || slots < 1 || slots > 64)
    return fail(SSPEC_ERR_INVALID_ARG, "chunk_pages must be in [1, 4096] and slots in [1, 64]");
  const size_t pb = sspec_offload_page_bytes(kv->num_kv_heads);
  const size_t table = sspec_offload_host_bytes(kv->num_kv_heads, chunk_pages, slots, 0);
  if (!dry) {
    if (!staging || staging_bytes < (size_t)slots * chunk_pages * pb)
      return fail(SSPEC_ERR_WORKSPACE, "staging buffer missing or smaller than slots*chunk_pages*%zu bytes", pb);
    if (!host) return fail(SSPEC_ERR_WORKSPACE, "host arena is NULL");
    if ((reinterpret_cast<uintptr_t>(staging) | reinterpret_cast<uintptr_t>(host)) % 256 != 0)
      return fail(SSPEC_ERR_WORKSPACE, "staging and host arena must be 256-byte aligned");
  }
  if (host_bytes < table + pb) return fail(SSPEC_ERR_WORKSPACE, "host arena holds no page (needs > %zu bytes)", table);
  sspec_offload* e = new (std::nothrow) sspec_offload();
  if (!e) return fail(SSPEC_ERR_INVALID_ARG, "out of host memory");
  e->kv = *kv;
  e->chunk_pages = chunk_pages;
  e->slots = slots;
  e->page_bytes = pb;
  e->staging = (uint8_t*)staging;
  e->host = (uint8_t*)host;
  e->host_pages = (host_bytes - table) / pb;
  e->ids = dry ? nullptr : (int32_t*)host;
  e->data = dry ? nullptr : (uint8_t*)host + table;   // planning-only: no host buffers
  e->side = (hipStream_t)side_stream;
  e->dry = dry;
  e->host_free.push_back({0, e->host_pages});
  for (int s = slots - 1; s >= 0; --s) e->free_slots.push_back(s);
  if (!dry) {
    e->ev.resize(slots);
    for (int s = 0; s < slots; ++s) {
      if (hipEventCreateWithFlags(&e->ev[s], hipEventDisableTiming) != hipSuccess) {
        for (int t = 0; t < s; ++t) (void)hipEventDestroy(e->ev[t]);
        delete e;
        return fail(SSPEC_ERR_HIP, "hipEventCreate failed");
      }
    }
  }
  *out = e;
  return SSPEC_OK;
}

int sspec_offload_destroy(sspec_offload* e) {
  if (!e) return SSPEC_OK;
  int rc = SSPEC_OK;
  if (!e->dry) {
    if (hipStreamSynchronize(e->side) != hipSuccess) rc = fail(SSPEC_ERR_HIP, "hipStreamSynchronize failed");
    for (auto& x : e->ev) (void)hipEventDestroy(x);
  }
  delete e;
  return rc;
}

int sspec_offload_evict(sspec_offload* e, int32_t req, const int32_t* pages, int32_t n_pages) {
  if (!e) return fail(SSPEC_ERR_INVALID_ARG, "engine is NULL");
  if (n_pages < 1 || !pages) return fail(SSPEC_ERR_INVALID_ARG, "evict needs n_pages >= 1 and a page list");
  if (find_home(e, req)) return fail(SSPEC_ERR_INVALID_ARG, "request %d already has a host copy", req);
  for (int32_t i = 0; i < n_pages; ++i)
    if (pages[i] < 0 || pages[i] >= e->kv.num_pages)
      return fail(SSPEC_ERR_INVALID_ARG, "page %d of request %d is outside [0, %d)", pages[i], req, e->kv.num_pages);
  const size_t at = host_alloc(e, (size_t)n_pages);
  if (at == SIZE_MAX) return fail(SSPEC_ERR_WORKSPACE, "host arena full (%d pages asked)", n_pages);
  OffloadJob j;
  j.req = req;
  j.kind = SSPEC_OFFLOAD_EVICT;
  j.pages.assign(pages, pages + n_pages);
  j.host_page = at;
  e->fifo.push_back(std::move(j));
  e->homes.push_back({req, at, n_pages});
  return SSPEC_OK;
}

int sspec_offload_restore(sspec_offload* e, int32_t req, const int32_t* pages, int32_t n_pages) {
  if (!e) return fail(SSPEC_ERR_INVALID_ARG, "engine is NULL");
  if (n_pages < 1 || !pages) return fail(SSPEC_ERR_INVALID_ARG, "restore needs n_pages >= 1 and a page list");
  const sspec_offload::Home* home = find_home(e, req);
  if (!home) return fail(SSPEC_ERR_INVALID_ARG, "request %d has no host copy", req);
  if (n_pages != home->n)
    return fail(SSPEC_ERR_INVALID_ARG, "request %d was evicted with %d pages, restore names %d", req, home->n, n_pages);
  for (auto& j : e->fifo)
    if (j.req == req && j.kind == SSPEC_OFFLOAD_RESTORE)
      return fail(SSPEC_ERR_INVALID_ARG, "request %d is already being restored", req);
  for (int32_t i = 0; i < n_pages; ++i)
    if (pages[i] < 0 || pages[i] >= e->kv.num_pages)
      return fail(SSPEC_ERR_INVALID_ARG, "page %d of request %d is outside [0, %d)", pages[i], req, e->kv.num_pages);
  OffloadJob j;
  j.req = req;
  j.kind = SSPEC_OFFLOAD_RESTORE;
  j.pages.assign(pages, pages + n_pages);
  j.host_page = home->at;
  e->fifo.push_back(std::move(j));
  return SSPEC_OK;
}

int sspec_offload_pump(sspec_offload* e, void* after_event, int32_t max_chunks) {
  if (!e) return fail(SSPEC_ERR_INVALID_ARG, "engine is NULL");
  if (max_chunks < 0) return fail(SSPEC_ERR_INVALID_ARG, "max_chunks must be >= 0");
  bool waited = false;
  for (auto& j : e->fifo) {
    while (max_chunks > 0 && j.issued < (int32_t)j.pages.size() && !e->free_slots.empty()) {
      if (!e->dry && after_event && !waited) {
        if (hipStreamWaitEvent(e->side, (hipEvent_t)after_event, 0) != hipSuccess)
          return fail(SSPEC_ERR_HIP, "hipStreamWaitEvent failed");
        waited = true;
      }
      const int32_t slot = e->free_slots.back();
      const int32_t first = j.issued;
      const int32_t count = std::min<int32_t>(e->chunk_pages, (int32_t)j.pages.size() - first);
      if (!e->dry) {
        int32_t* ids = e->ids + (size_t)slot * e->chunk_pages;
        std::memcpy(ids, j.pages.data() + first, sizeof(int32_t) * (size_t)count);
        uint16_t* stage = (uint16_t*)(e->staging + (size_t)slot * e->chunk_pages * e->page_bytes);
        uint8_t* hp = e->data + (j.host_page + (size_t)first) * e->page_bytes;
        const size_t bytes = (size_t)count * e->page_bytes;
        int rc;
        if (j.kind == SSPEC_OFFLOAD_EVICT) {
          if ((rc = launch_move(true, &e->kv, ids, count, stage, nullptr, e->side))) return rc;
          if (hipMemcpyAsync(hp, stage, bytes, hipMemcpyDeviceToHost, e->side) != hipSuccess)
            return fail(SSPEC_ERR_HIP, "hipMemcpyAsync (device to host) failed");
        } else {
          if (hipMemcpyAsync(stage, hp, bytes, hipMemcpyHostToDevice, e->side) != hipSuccess)
            return fail(SSPEC_ERR_HIP, "hipMemcpyAsync (host to device) failed");
          if ((rc = launch_move(false, &e->kv, ids, count, stage, nullptr, e->side))) return rc;
        }
        if (hipEventRecord(e->ev[slot], e->side) != hipSuccess) return fail(SSPEC_ERR_HIP, "hipEventRecord failed");
      }
      e->free_slots.pop_back();
      e->inflight.push_back({&j, first, count, slot});
      e->trace.insert(e->trace.end(), {j.req, j.kind, first, count});
      j.issued += count;
      ++j.chunks_left;
      --max_chunks;
    }
    // FIFO: a later job starts only once every chunk of this one is issued
    if (j.issued < (int32_t)j.pages.size()) break;
  }
  return SSPEC_OK;
}

int sspec_offload_poll(sspec_offload* e, int32_t* reqs, int32_t* kinds, int32_t cap, int32_t* n_done) {
  if (!e || !n_done) return fail(SSPEC_ERR_INVALID_ARG, "engine or n_done is NULL");
  if (cap < 0 || (cap > 0 && (!reqs || !kinds))) return fail(SSPEC_ERR_INVALID_ARG, "bad output arrays");
  *n_done = 0;
  // chunks finish in issue order (one stream): retire from the front
  while (!e->inflight.empty()) {
    OffloadChunk& c = e->inflight.front();
    if (!e->dry) {
      const hipError_t q = hipEventQuery(e->ev[c.slot]);
      if (q == hipErrorNotReady) break;
      if (q != hipSuccess) return fail(SSPEC_ERR_HIP, "hipEventQuery failed");
    }
    e->free_slots.push_back(c.slot);
    --c.job->chunks_left;
    e->inflight.pop_front();
  }
  // jobs retire in FIFO order once all their chunks are issued and finished
  while (!e->fifo.empty() && *n_done < cap) {
    OffloadJob& j = e->fifo.front();
    if (j.issued < (int32_t)j.pages.size() || j.chunks_left > 0) break;
    if (j.kind == SSPEC_OFFLOAD_RESTORE) {
      // the host copy is free again
      for (size_t i = 0; i < e->homes.size(); ++i)
        if (e->homes[i].req == j.req) {
          host_free(e, e->homes[i].at, (size_t)e->homes[i].n);
          e->homes.erase(e->homes.begin() + (long)i);
          break;
        }
    }
    reqs[*n_done] = j.req;
    kinds[*n_done] = j.kind;
    ++*n_done;
    e->fifo.pop_front();
  }
  return SSPEC_OK;
}

int sspec_offload_pending(const sspec_offload* e, int32_t* jobs, int32_t* chunks_in_flight, int64_t* host_pages_free) {
  if (!e) return fail(SSPEC_ERR_INVALID_ARG, "engine is NULL");
  if (jobs) *jobs = (int32_t)e->fifo.size();
  if (chunks_in_flight) *chunks_in_flight = (int32_t)e->inflight.size();
  if (host_pages_free) {
    size_t f = 0;
    for (auto& x : e->host_free) f += x.second;
    *host_pages_free = (int64_t)f;
  }
  return SSPEC_OK;
}

int sspec_offload_trace(const sspec_offload* e, int32_t* out, int32_t cap, int32_t* n) {
  if (!e || !n) return fail(SSPEC_ERR_INVALID_ARG, "engine or n is NULL");
  const int32_t m = (int32_t)(e->trace.size() / 4);
  *n = m;
  if (out) std::memcpy(out, e->trace.data(), sizeof(int32_t) * 4 * (size_t)std::min(std::max(cap, 0), m));
  return SSPEC_OK;
}

}  // extern "C"

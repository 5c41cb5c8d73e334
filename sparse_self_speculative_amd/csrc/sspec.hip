// C ABI of the SparseSpec attention hot path on MI355X (gfx950), declared in
// include/sspec.h: argument validation, workspace layout, and the launch of
// the persistent kernel (kernel.hpp) over pieces of at most kMaxItems items.
//
// Method: talk notes "Accelerating Large-Scale Reasoning Model Inference
// with Sparse Self-Speculative Decoding" (MLSys 2026), sections PillarAttn
// (paper §4.1) and Unified batch scheduler (paper §4.2, §5.6 Fig. 15).
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

#include "kernel.hpp"

namespace sspec {

#define SSPEC_DECL_ROW(g) std::array<KernelFn, 8> kernel_table_g##g(); const char* build_config_g##g();
SSPEC_DECL_ROW(1) SSPEC_DECL_ROW(2) SSPEC_DECL_ROW(3) SSPEC_DECL_ROW(4)
SSPEC_DECL_ROW(5) SSPEC_DECL_ROW(6) SSPEC_DECL_ROW(7) SSPEC_DECL_ROW(8)
#undef SSPEC_DECL_ROW

// Workspace initialisation: every word zero except the header's magic and
// clean_end (the whole workspace is zero, so every layout's zone is clean).
__global__ void ws_init_kernel(uint32_t* p, size_t n, uint64_t clean_end) {
  constexpr size_t kMagicW = offsetof(WsHeader, magic) / 4, kCleanW = offsetof(WsHeader, clean_end) / 4;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
    uint32_t v = 0u;
    if (i == kMagicW) v = kWsMagic;
    if (i == kCleanW) v = (uint32_t)clean_end;
    if (i == kCleanW + 1) v = (uint32_t)(clean_end >> 32);
    p[i] = v;
  }
}

// Zero-state zone of a layout: words [b, e) of the workspace are cleared and
// the header's clean_end set to e (words).  Only the header word is written
// outside the zone, by one thread.
__global__ void ws_zone_kernel(uint32_t* p, size_t b, size_t e) {
  for (size_t i = b + blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < e; i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
  if (blockIdx.x == 0 && threadIdx.x == 0)
    reinterpret_cast<WsHeader*>(p)->clean_end = (uint64_t)e * 4;
}

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

constexpr int kMaxKvHeads = 256;

int check_heads(int hq, int hkv, int k) {
  if (hkv < 1 || hq < 1) return fail(SSPEC_ERR_INVALID_ARG, "num_q_heads and num_kv_heads must be >= 1 (got %d, %d)", hq, hkv);
  if (hkv > kMaxKvHeads) return fail(SSPEC_ERR_UNSUPPORTED, "num_kv_heads must be <= %d (got %d)", kMaxKvHeads, hkv);
  if (hq % hkv != 0) return fail(SSPEC_ERR_UNSUPPORTED, "num_q_heads (%d) must be a multiple of num_kv_heads (%d)", hq, hkv);
  const int G = hq / hkv;
  if (G > kMaxG) return fail(SSPEC_ERR_UNSUPPORTED, "GQA group size %d > %d", G, kMaxG);
  if (k < 0 || k > kMaxK) return fail(SSPEC_ERR_UNSUPPORTED, "k must be in [0, %d] (got %d)", kMaxK, k);
  if (G * (k + 1) > kMaxRows) return fail(SSPEC_ERR_UNSUPPORTED, "G*(k+1) = %d > %d", G * (k + 1), kMaxRows);
  return SSPEC_OK;
}

int check_ctx(int max_ctx) {
  if (max_ctx < 1 || max_ctx > kMaxCtx) return fail(SSPEC_ERR_UNSUPPORTED, "max_ctx must be in [1, %d] (got %d)", kMaxCtx, max_ctx);
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
  if ((reinterpret_cast<uintptr_t>(kv->k_pages) | reinterpret_cast<uintptr_t>(kv->v_pages)) % 16 != 0)
    return fail(SSPEC_ERR_INVALID_ARG, "k_pages and v_pages must be 16-byte aligned");
  // row ids (page * num_kv_heads + h) * 16 + slot are 32-bit
  if ((int64_t)kv->num_pages * kv->num_kv_heads * kPage > 0xffffffffLL)
    return fail(SSPEC_ERR_UNSUPPORTED, "num_pages * num_kv_heads * 16 must fit in 32 bits");
  return SSPEC_OK;
}

int check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (!ws) return fail(SSPEC_ERR_WORKSPACE, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(ws) % 256 != 0) return fail(SSPEC_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (ws_bytes < need) return fail(SSPEC_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", ws_bytes, need);
  return SSPEC_OK;
}

std::mutex g_occ_mu;
std::unordered_map<uint64_t, int> g_grid_cache;

// Per (device, workspace address): how far the workspace's zero prefix
// [kZoneBegin, clean_end) reaches after the work enqueued on it so far (the
// device header holds the same value once that work has run).  Calls that
// share a workspace are ordered, so the host sees them in stream order.  An
// entry is only a cache: a missing one makes the next call clear its zone.
std::mutex g_ws_mu;
std::unordered_map<uint64_t, size_t> g_ws_clean;
constexpr size_t kWsCacheMax = 4096;

int ws_key(const void* ws, uint64_t* key) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(SSPEC_ERR_HIP, "hipGetDevice failed");
  *key = (uint64_t)reinterpret_cast<uintptr_t>(ws) ^ ((uint64_t)dev << 56);
  return SSPEC_OK;
}

void ws_cache_set(uint64_t key, size_t clean_end) {
  std::lock_guard<std::mutex> lk(g_ws_mu);
  if (g_ws_clean.size() >= kWsCacheMax) g_ws_clean.clear();
  g_ws_clean[key] = clean_end;
}

// Before a launch with layout wl: clear the zone unless the cache says it is
// clean; afterwards only [kZoneBegin, wl.zone_end) is known to be zero (the
// data regions that follow may now hold anything).
int ws_prepare(void* ws, const WsLayout& wl, hipStream_t st) {
  uint64_t key;
  int rc = ws_key(ws, &key);
  if (rc) return rc;
  size_t clean = 0;
  {
    std::lock_guard<std::mutex> lk(g_ws_mu);
    auto f = g_ws_clean.find(key);
    if (f != g_ws_clean.end()) clean = f->second;
  }
  if (clean < wl.zone_end) {
    const size_t b = kZoneBegin / 4, e = wl.zone_end / 4;
    const int grid = (int)std::max<size_t>(1, std::min<size_t>((e - b + 255) / 256, 2048));
    hipLaunchKernelGGL(ws_zone_kernel, dim3(grid), dim3(256), 0, st, (uint32_t*)ws, b, e);
    if ((rc = check_launch("ws_zone_kernel"))) return rc;
  }
  ws_cache_set(key, wl.zone_end);
  return SSPEC_OK;
}

// Every kernel object must come from one configuration of the build macros
// (they fix chunk sizes and the workspace layout): checked once, before the
// first launch.
int check_build() {
  static const std::string bad = [] {
    const char* (*cfg[8])() = {build_config_g1, build_config_g2, build_config_g3, build_config_g4,
                               build_config_g5, build_config_g6, build_config_g7, build_config_g8};
    const std::string mine = build_config();
    for (int g = 0; g < 8; ++g)
      if (mine != cfg[g]())
        return "kernel objects of G=" + std::to_string(g + 1) + " were built with \"" + cfg[g]() +
               "\", the host code with \"" + mine + "\"";
    return std::string();
  }();
  if (!bad.empty()) return fail(SSPEC_ERR_UNSUPPORTED, "mixed build: %s", bad.c_str());
  return SSPEC_OK;
}

int resident_grid(uint64_t key, const void* kernel, int threads, int* grid) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(SSPEC_ERR_HIP, "hipGetDevice failed");
  key |= (uint64_t)dev << 32;
  {
    std::lock_guard<std::mutex> lk(g_occ_mu);
    auto f = g_grid_cache.find(key);
    if (f != g_grid_cache.end()) {
      *grid = f->second;
      return SSPEC_OK;
    }
  }
  int cus = 0, occ = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return fail(SSPEC_ERR_HIP, "hipDeviceGetAttribute failed");
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, threads, 0) != hipSuccess)
    return fail(SSPEC_ERR_HIP, "hipOccupancyMaxActiveBlocksPerMultiprocessor failed");
  *grid = cus * (occ > 0 ? occ : 1);
  std::lock_guard<std::mutex> lk(g_occ_mu);
  g_grid_cache[key] = *grid;
  return SSPEC_OK;
}

const std::array<KernelFn, 8>& kernel_rows(int g) {
  static const std::array<KernelFn, 8> rows[8] = {kernel_table_g1(), kernel_table_g2(), kernel_table_g3(),
                                                  kernel_table_g4(), kernel_table_g5(), kernel_table_g6(),
                                                  kernel_table_g7(), kernel_table_g8()};
  return rows[g];
}

int run(const Job& p, int G, int nqt, hipStream_t st) {
  KernelFn fn = nullptr;
  if (G >= 1 && G <= 8 && nqt >= 1 && nqt <= 8) fn = kernel_rows(G - 1)[nqt - 1];
  if (!fn) {
    // a selection-only launch runs on any instance
    if (p.mode == kModeTopk)
      for (int g = 0; g < 8 && !fn; ++g)
        for (int t = 0; t < 8 && !fn; ++t) fn = kernel_rows(g)[t];
    if (!fn) return fail(SSPEC_ERR_UNSUPPORTED, "no kernel built for G=%d, %d query tiles", G, nqt);
  }
  return fn(p, st);
}

// Launch over items in pieces of at most kMaxItems (item arrays are
// advanced by the caller through `shift`); every piece uses the layout of
// p.layout_n items.
template <class Shift>
int run_pieces(Job p, const WsLayout& wl, int G, int nqt, hipStream_t st, Shift shift) {
  int rc = check_build();
  if (rc) return rc;
  if ((rc = ws_prepare(p.ws, wl, st))) return rc;
  const int n = p.n;
  for (int i0 = 0; i0 < n; i0 += kMaxItems) {
    Job q = p;
    q.n = std::min(kMaxItems, n - i0);
    shift(q, i0);
    const int rc = run(q, G, nqt, st);
    if (rc) return rc;
  }
  return SSPEC_OK;
}

// ------------------------------------------- static scratch (no allocation)
// The workspace of sspec_pillar_topk_noalloc: one array per device, part of
// the library's code object, alive until the process ends.  In host code
// `scratch` names a host-side stand-in, never a device address: its device
// address comes from hipGetSymbolAddress, once per device, and only that
// address is ever passed to a kernel.  Every call on one device shares it
// (calls that overlap on one device race); the zero-state zone protocol of
// the workspace (WsLayout) clears what must start at zero.
constexpr size_t kScratchBytes = (size_t)64 << 20;
std::mutex g_scratch_mu;
std::unordered_map<int, void*> g_scratch_ptr;   // device -> device address of `scratch`

}  // namespace sspec

static __device__ __align__(256) uint8_t scratch[sspec::kScratchBytes];

namespace sspec {

// This device's scratch address; the first call on a device looks it up and
// clears the array (one fill kernel on `st`).  Allocates nothing.
int scratch_for_device(hipStream_t st, void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(SSPEC_ERR_HIP, "hipGetDevice failed");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  auto f = g_scratch_ptr.find(dev);
  if (f != g_scratch_ptr.end()) {
    *out = f->second;
    return SSPEC_OK;
  }
  void* ptr = nullptr;
  const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess || ptr == nullptr)
    return fail(SSPEC_ERR_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev, hipGetErrorString(e));
  const size_t n = kScratchBytes / 4;
  hipLaunchKernelGGL(ws_init_kernel, dim3(4096), dim3(256), 0, st, (uint32_t*)ptr, n, (uint64_t)kScratchBytes);
  int rc = check_launch("ws_init_kernel");
  if (rc) return rc;
  uint64_t key;
  if ((rc = ws_key(ptr, &key))) return rc;
  ws_cache_set(key, kScratchBytes);
  g_scratch_ptr[dev] = ptr;
  *out = ptr;
  return SSPEC_OK;
}

// sspec_pillar_topk and its allocation-free variant (scratch: the workspace
// is this device's static scratch array instead of ws/ws_bytes).
int pillar_topk_impl(const float* logits, const float* lse, int64_t logit_stride, const int32_t* seq_ids,
                     const int32_t* ctx_lens, int32_t n, int32_t num_seqs, int32_t max_ctx, int32_t num_q_heads,
                     int32_t num_kv_heads, int32_t k, double s, int32_t* sel_idx, int32_t sel_stride,
                     int32_t* sel_count, int32_t* sel_len, void* ws, size_t ws_bytes, void* stream, bool scratch) {
  int rc;
  if ((rc = check_heads(num_q_heads, num_kv_heads, k))) return rc;
  if ((rc = check_ctx(max_ctx))) return rc;
  if (n < 0 || num_seqs < 1) return fail(SSPEC_ERR_INVALID_ARG, "bad sizes (n %d, num_seqs %d)", n, num_seqs);
  if (!(s > 0.0 && s <= 1.0)) return fail(SSPEC_ERR_INVALID_ARG, "s must be in (0, 1] (got %g)", s);
  if (n == 0) return SSPEC_OK;
  if (!logits || !lse || !seq_ids || !ctx_lens || !sel_idx || !sel_count || !sel_len)
    return fail(SSPEC_ERR_INVALID_ARG, "a pillar_topk array pointer is NULL");
  if (logit_stride < round_up(max_ctx, kPage) || logit_stride > kMaxCtx + kPage || logit_stride % kPage != 0)
    return fail(SSPEC_ERR_INVALID_ARG, "logit_stride (%lld) must be a multiple of 16 in [round_up(max_ctx, 16), %d]",
                (long long)logit_stride, kMaxCtx + kPage);
  if (reinterpret_cast<uintptr_t>(logits) % 16 != 0)
    return fail(SSPEC_ERR_INVALID_ARG, "logits must be 16-byte aligned");
  const int G = num_q_heads / num_kv_heads, kp1 = k + 1;
  if (sel_stride < select_count(max_ctx, s))
    return fail(SSPEC_ERR_INVALID_ARG, "sel_stride (%d) < ceil(s*max_ctx) = %d", sel_stride, select_count(max_ctx, s));
  const int ln = std::min<int>(n, kMaxItems);
  const WsLayout wl(kModeTopk, ln, 0, max_ctx, num_kv_heads, num_kv_heads, 0);
  if (scratch) {
    if (wl.total > kScratchBytes)
      return fail(SSPEC_ERR_WORKSPACE,
                  "this call needs %zu bytes of workspace, more than the %zu-byte static scratch of "
                  "sspec_pillar_topk_noalloc (use sspec_pillar_topk with a workspace)", wl.total, kScratchBytes);
    if ((rc = scratch_for_device((hipStream_t)stream, &ws))) return rc;
    ws_bytes = kScratchBytes;
  }
  if ((rc = check_ws(ws, ws_bytes, wl.total))) return rc;
  Job p{};
  p.mode = kModeTopk;
  p.layout_n = ln;
  p.seq_ids = seq_ids;
  p.ctx_lens = ctx_lens;
  p.n = n;
  p.num_seqs = num_seqs;
  p.max_ctx = max_ctx;
  p.hq = num_q_heads;
  p.hkv = num_kv_heads;
  p.k = k;
  p.s = s;
  p.logits = const_cast<float*>(logits);
  p.lse_in = lse;
  p.lstride = logit_stride;
  p.sel_idx = sel_idx;
  p.sel_stride = sel_stride;
  p.sel_count = sel_count;
  p.sel_len = sel_len;
  p.ws = (uint8_t*)ws;
  p.ws_bytes = ws_bytes;
  // the score math needs the group size G as a kernel constant
  return run_pieces(p, wl, G, 1, (hipStream_t)stream, [&](Job& j, int i0) {
    j.seq_ids += i0;
    j.logits += (int64_t)i0 * num_kv_heads * logit_stride * round_up(G * kp1, 4);
    j.lse_in += (int64_t)i0 * kp1 * num_q_heads;
  });
}

}  // namespace sspec

using namespace sspec;

// ==================================================================== ABI ===
extern "C" {

const char* sspec_last_error(void) { return g_last_error.c_str(); }

int sspec_workspace_init(void* ws, size_t ws_bytes, void* stream) {
  if (!ws) return fail(SSPEC_ERR_WORKSPACE, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(ws) % 256 != 0) return fail(SSPEC_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (ws_bytes < kZoneBegin) return fail(SSPEC_ERR_WORKSPACE, "workspace smaller than its %zu-byte header", kZoneBegin);
  uint64_t key;
  int rc = ws_key(ws, &key);
  if (rc) return rc;
  const size_t n = ws_bytes / 4;
  const int grid = (int)std::min<size_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(ws_init_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, (uint32_t*)ws, n,
                     (uint64_t)(n * 4));
  if ((rc = check_launch("ws_init_kernel"))) return rc;
  ws_cache_set(key, n * 4);
  return SSPEC_OK;
}

int sspec_read_device_error(void* ws, int clear, void* stream, uint32_t* flags) {
  if (!ws || !flags) return fail(SSPEC_ERR_INVALID_ARG, "ws and flags must not be NULL");
  hipStream_t st = (hipStream_t)stream;
  if (hipStreamSynchronize(st) != hipSuccess) return fail(SSPEC_ERR_HIP, "hipStreamSynchronize failed");
  uint32_t v = 0;
  if (hipMemcpy(&v, ws, sizeof(v), hipMemcpyDeviceToHost) != hipSuccess) return fail(SSPEC_ERR_HIP, "hipMemcpy failed");
  *flags = v;
  if (v & (SSPEC_DEV_ERR_WAIT_TIMEOUT | SSPEC_DEV_ERR_WS_STATE)) {
    // stale state may be left in the zone: the next call clears it
    uint64_t key;
    if (ws_key(ws, &key) == SSPEC_OK) {
      std::lock_guard<std::mutex> lk(g_ws_mu);
      g_ws_clean.erase(key);
    }
  }
  if (clear) {
    const uint32_t z = 0;
    if (hipMemcpy(ws, &z, sizeof(z), hipMemcpyHostToDevice) != hipSuccess) return fail(SSPEC_ERR_HIP, "hipMemcpy failed");
  }
  return SSPEC_OK;
}

size_t sspec_verify_workspace_size(int32_t n, int32_t max_ctx, int32_t num_q_heads, int32_t num_kv_heads, int32_t k) {
  if (n < 0 || max_ctx < 1 || max_ctx > kMaxCtx || num_kv_heads < 1 || num_q_heads < num_kv_heads || k < 0) return 0;
  return WsLayout(kModeVerify, std::min<int>(n, kMaxItems), 0, max_ctx, num_q_heads, num_kv_heads, k).total;
}

int sspec_verify_attn(const sspec_paged_kv* kv, const uint16_t* q, const int32_t* seq_ids, const int32_t* ctx_lens,
                      int32_t n, int32_t max_ctx, int32_t num_q_heads, int32_t k, float sm_scale, uint16_t* out,
                      float* lse, float* logits, int64_t logit_stride, void* ws, size_t ws_bytes, void* stream) {
  int rc;
  if ((rc = check_kv(kv))) return rc;
  if ((rc = check_heads(num_q_heads, kv->num_kv_heads, k))) return rc;
  if ((rc = check_ctx(max_ctx))) return rc;
  if (n < 0) return fail(SSPEC_ERR_INVALID_ARG, "n must be >= 0 (got %d)", n);
  if (!std::isfinite(sm_scale)) return fail(SSPEC_ERR_INVALID_ARG, "sm_scale must be finite");
  if (n == 0) return SSPEC_OK;
  if (!q || !seq_ids || !ctx_lens || !out || !lse || !logits) return fail(SSPEC_ERR_INVALID_ARG, "a verify array pointer is NULL");
  if (logit_stride < round_up(max_ctx, kPage) || logit_stride > kMaxCtx + kPage || logit_stride % kPage != 0)
    return fail(SSPEC_ERR_INVALID_ARG, "logit_stride (%lld) must be a multiple of 16 in [round_up(max_ctx, 16) = %d, %d]",
                (long long)logit_stride, round_up(max_ctx, kPage), kMaxCtx + kPage);
  if (reinterpret_cast<uintptr_t>(logits) % 16 != 0 || reinterpret_cast<uintptr_t>(q) % 16 != 0 ||
      reinterpret_cast<uintptr_t>(out) % 16 != 0)
    return fail(SSPEC_ERR_INVALID_ARG, "q, out and logits must be 16-byte aligned");
  const int hkv = kv->num_kv_heads;
  const int ln = std::min<int>(n, kMaxItems);
  const WsLayout wl(kModeVerify, ln, 0, max_ctx, num_q_heads, hkv, k);
  if ((rc = check_ws(ws, ws_bytes, wl.total))) return rc;
  const int G = num_q_heads / hkv, kp1 = k + 1;
  Job p{};
  p.mode = kModeVerify;
  p.layout_n = ln;
  p.kv = *kv;
  p.q = q;
  p.seq_ids = seq_ids;
  p.ctx_lens = ctx_lens;
  p.n = n;
  p.num_seqs = kv->num_seqs;
  p.max_ctx = max_ctx;
  p.hq = num_q_heads;
  p.hkv = hkv;
  p.k = k;
  p.scale = sm_scale;
  p.logits = logits;
  p.lstride = logit_stride;
  p.out = out;
  p.lse = lse;
  p.ws = (uint8_t*)ws;
  p.ws_bytes = ws_bytes;
  return run_pieces(p, wl, G, cdiv(G * kp1, 16), (hipStream_t)stream, [&](Job& j, int i0) {
    j.q += (int64_t)i0 * kp1 * num_q_heads * kD;
    j.seq_ids += i0;
    j.out += (int64_t)i0 * kp1 * num_q_heads * kD;
    j.lse += (int64_t)i0 * kp1 * num_q_heads;
    j.logits += (int64_t)i0 * hkv * logit_stride * round_up(G * kp1, 4);
  });
}

size_t sspec_pillar_topk_workspace_size(int32_t n, int32_t max_ctx, int32_t num_kv_heads) {
  if (n < 0 || max_ctx < 1 || max_ctx > kMaxCtx || num_kv_heads < 1) return 0;
  return WsLayout(kModeTopk, std::min<int>(n, kMaxItems), 0, max_ctx, num_kv_heads, num_kv_heads, 0).total;
}

int sspec_pillar_topk(const float* logits, const float* lse, int64_t logit_stride, const int32_t* seq_ids,
                      const int32_t* ctx_lens, int32_t n, int32_t num_seqs, int32_t max_ctx, int32_t num_q_heads,
                      int32_t num_kv_heads, int32_t k, double s, int32_t* sel_idx, int32_t sel_stride,
                      int32_t* sel_count, int32_t* sel_len, void* ws, size_t ws_bytes, void* stream) {
  return pillar_topk_impl(logits, lse, logit_stride, seq_ids, ctx_lens, n, num_seqs, max_ctx, num_q_heads,
                          num_kv_heads, k, s, sel_idx, sel_stride, sel_count, sel_len, ws, ws_bytes, stream, false);
}

int sspec_pillar_topk_noalloc(const float* logits, const float* lse, int64_t logit_stride, const int32_t* seq_ids,
                              const int32_t* ctx_lens, int32_t n, int32_t num_seqs, int32_t max_ctx,
                              int32_t num_q_heads, int32_t num_kv_heads, int32_t k, double s, int32_t* sel_idx,
                              int32_t sel_stride, int32_t* sel_count, int32_t* sel_len, void* stream) {
  return pillar_topk_impl(logits, lse, logit_stride, seq_ids, ctx_lens, n, num_seqs, max_ctx, num_q_heads,
                          num_kv_heads, k, s, sel_idx, sel_stride, sel_count, sel_len, nullptr, 0, stream, true);
}

size_t sspec_draft_workspace_size(int32_t n, int32_t max_ctx, int32_t num_q_heads, int32_t num_kv_heads) {
  if (n < 0 || max_ctx < 1 || max_ctx > kMaxCtx || num_kv_heads < 1 || num_q_heads < num_kv_heads) return 0;
  return WsLayout(kModeDraft, std::min<int>(n, kMaxItems), 0, max_ctx, num_q_heads, num_kv_heads, 0).total;
}

int sspec_sparse_draft_attn(const sspec_paged_kv* kv, const uint16_t* q, const int32_t* seq_ids, const int32_t* ctx_lens,
                            const int32_t* sel_idx, int32_t sel_stride, const int32_t* sel_count, const int32_t* sel_len,
                            int32_t n, int32_t max_ctx, int32_t num_q_heads, float sm_scale, uint16_t* out, float* lse,
                            void* ws, size_t ws_bytes, void* stream) {
  int rc;
  if ((rc = check_kv(kv))) return rc;
  if ((rc = check_heads(num_q_heads, kv->num_kv_heads, 0))) return rc;
  if ((rc = check_ctx(max_ctx))) return rc;
  if (n < 0 || sel_stride < 0) return fail(SSPEC_ERR_INVALID_ARG, "bad sizes (n %d, sel_stride %d)", n, sel_stride);
  if (!std::isfinite(sm_scale)) return fail(SSPEC_ERR_INVALID_ARG, "sm_scale must be finite");
  if (n == 0) return SSPEC_OK;
  if (!q || !seq_ids || !ctx_lens || !sel_count || !sel_len || !out || (!sel_idx && sel_stride > 0))
    return fail(SSPEC_ERR_INVALID_ARG, "a draft array pointer is NULL");
  if (reinterpret_cast<uintptr_t>(q) % 16 != 0 || reinterpret_cast<uintptr_t>(out) % 16 != 0)
    return fail(SSPEC_ERR_INVALID_ARG, "q and out must be 16-byte aligned");
  const int hkv = kv->num_kv_heads;
  const int ln = std::min<int>(n, kMaxItems);
  const WsLayout wl(kModeDraft, ln, 0, max_ctx, num_q_heads, hkv, 0);
  if ((rc = check_ws(ws, ws_bytes, wl.total))) return rc;
  Job p{};
  p.mode = kModeDraft;
  p.layout_n = ln;
  p.kv = *kv;
  p.q = q;
  p.seq_ids = seq_ids;
  p.ctx_lens = ctx_lens;
  p.n = n;
  p.num_seqs = kv->num_seqs;
  p.max_ctx = max_ctx;
  p.hq = num_q_heads;
  p.hkv = hkv;
  p.k = 0;
  p.scale = sm_scale;
  p.sel_idx = const_cast<int32_t*>(sel_idx);
  p.sel_stride = sel_stride;
  p.sel_count = const_cast<int32_t*>(sel_count);
  p.sel_len = const_cast<int32_t*>(sel_len);
  p.out = out;
  p.lse = lse;
  p.ws = (uint8_t*)ws;
  p.ws_bytes = ws_bytes;
  const int G = num_q_heads / hkv;
  return run_pieces(p, wl, G, 1, (hipStream_t)stream, [&](Job& j, int i0) {
    j.q += (int64_t)i0 * num_q_heads * kD;
    j.seq_ids += i0;
    j.out += (int64_t)i0 * num_q_heads * kD;
    if (j.lse) j.lse += (int64_t)i0 * num_q_heads;
  });
}

size_t sspec_unified_workspace_size(int32_t num_seqs, int32_t max_verify, int32_t max_ctx, int32_t num_q_heads,
                                    int32_t num_kv_heads, int32_t k) {
  if (num_seqs < 1 || num_seqs > kMaxItems || max_verify < 0 || max_ctx < 1 || max_ctx > kMaxCtx || num_kv_heads < 1 ||
      num_q_heads < num_kv_heads || k < 0)
    return 0;
  return WsLayout(kModeUnified, num_seqs, std::min(max_verify, num_seqs), max_ctx, num_q_heads, num_kv_heads, k).total;
}

}  // extern "C"

namespace sspec {
int unified_impl(const sspec_paged_kv* kv, const uint16_t* q, const int32_t* ctx_lens, const int32_t* bucket_ids,
                 int32_t verify_bucket, int32_t num_seqs, int32_t max_verify, int32_t max_ctx, int32_t num_q_heads,
                 int32_t k, double s, float sm_scale, int32_t* sel_idx, int32_t sel_stride, int32_t* sel_count,
                 int32_t* sel_len, uint16_t* out, float* lse, void* ws, size_t ws_bytes, void* stream, int naive,
                 const int32_t* seq_ids, int32_t num_slots) {
  int rc;
  if ((rc = check_kv(kv))) return rc;
  if ((rc = check_heads(num_q_heads, kv->num_kv_heads, k))) return rc;
  if ((rc = check_ctx(max_ctx))) return rc;
  if (num_seqs < 1 || num_seqs > kMaxItems)
    return fail(SSPEC_ERR_UNSUPPORTED, "num_seqs must be in [1, %d] (got %d)", kMaxItems, num_seqs);
  if (num_seqs > kv->num_seqs) return fail(SSPEC_ERR_INVALID_ARG, "num_seqs (%d) > kv->num_seqs (%d)", num_seqs, kv->num_seqs);
  if (max_verify < 0) return fail(SSPEC_ERR_INVALID_ARG, "max_verify must be >= 0 (got %d)", max_verify);
  if (!(s > 0.0 && s <= 1.0)) return fail(SSPEC_ERR_INVALID_ARG, "s must be in (0, 1] (got %g)", s);
  if (!std::isfinite(sm_scale)) return fail(SSPEC_ERR_INVALID_ARG, "sm_scale must be finite");
  if (!q || !ctx_lens || !bucket_ids || !sel_idx || !sel_count || !sel_len || !out || !lse)
    return fail(SSPEC_ERR_INVALID_ARG, "a unified array pointer is NULL");
  if (reinterpret_cast<uintptr_t>(q) % 16 != 0 || reinterpret_cast<uintptr_t>(out) % 16 != 0)
    return fail(SSPEC_ERR_INVALID_ARG, "q and out must be 16-byte aligned");
  if (sel_stride < select_count(max_ctx, s))
    return fail(SSPEC_ERR_INVALID_ARG, "sel_stride (%d) < ceil(s*max_ctx) = %d", sel_stride, select_count(max_ctx, s));
  const int hkv = kv->num_kv_heads;
  // by slot, the workspace is carved for the slot count (the batch size may
  // change from launch to launch without a new layout)
  const int layout_n = seq_ids ? std::min(num_slots, kMaxItems) : num_seqs;
  const int mv = std::min(max_verify, layout_n);
  const WsLayout wl(kModeUnified, layout_n, mv, max_ctx, num_q_heads, hkv, k);
  if ((rc = check_ws(ws, ws_bytes, wl.total))) return rc;
  Job p{};
  p.mode = kModeUnified;
  p.naive = naive;
  p.layout_n = layout_n;
  p.kv = *kv;
  p.q = q;
  p.ctx_lens = ctx_lens;
  p.bucket_ids = bucket_ids;
  p.verify_bucket = verify_bucket;
  p.n = num_seqs;
  p.num_seqs = seq_ids ? num_slots : num_seqs;
  p.seq_ids = seq_ids;
  p.max_verify = mv;
  p.max_ctx = max_ctx;
  p.hq = num_q_heads;
  p.hkv = hkv;
  p.k = k;
  p.s = s;
  p.scale = sm_scale;
  p.sel_idx = sel_idx;
  p.sel_stride = sel_stride;
  p.sel_count = sel_count;
  p.sel_len = sel_len;
  p.out = out;
  p.lse = lse;
  p.ws = (uint8_t*)ws;
  p.ws_bytes = ws_bytes;
  const int G = num_q_heads / hkv;
  const int nqt = cdiv(G * (k + 1), 16);
  if (naive && nqt > 3)
    return fail(SSPEC_ERR_UNSUPPORTED, "naive batching needs G*(k+1) <= 48 (got %d)", G * (k + 1));
  return run_pieces(p, wl, G, nqt, (hipStream_t)stream, [](Job&, int) {});
}
}  // namespace sspec

extern "C" {

int sspec_unified_attn(const sspec_paged_kv* kv, const uint16_t* q, const int32_t* ctx_lens, const int32_t* bucket_ids,
                       int32_t verify_bucket, int32_t num_seqs, int32_t max_verify, int32_t max_ctx, int32_t num_q_heads,
                       int32_t k, double s, float sm_scale, int32_t* sel_idx, int32_t sel_stride, int32_t* sel_count,
                       int32_t* sel_len, uint16_t* out, float* lse, void* ws, size_t ws_bytes, void* stream) {
  return unified_impl(kv, q, ctx_lens, bucket_ids, verify_bucket, num_seqs, max_verify, max_ctx, num_q_heads, k, s,
                      sm_scale, sel_idx, sel_stride, sel_count, sel_len, out, lse, ws, ws_bytes, stream, 0, nullptr, 0);
}

int sspec_unified_attn_slots(const sspec_paged_kv* kv, const uint16_t* q, const int32_t* seq_ids,
                             const int32_t* ctx_lens, const int32_t* bucket_ids, int32_t verify_bucket,
                             int32_t num_items, int32_t max_verify, int32_t max_ctx, int32_t num_q_heads, int32_t k,
                             double s, float sm_scale, int32_t* sel_idx, int32_t sel_stride, int32_t* sel_count,
                             int32_t* sel_len, uint16_t* out, float* lse, void* ws, size_t ws_bytes, void* stream) {
  if (!seq_ids) return fail(SSPEC_ERR_INVALID_ARG, "seq_ids is NULL");
  if (!kv) return fail(SSPEC_ERR_INVALID_ARG, "kv is NULL");
  return unified_impl(kv, q, ctx_lens, bucket_ids, verify_bucket, num_items, max_verify, max_ctx, num_q_heads, k, s,
                      sm_scale, sel_idx, sel_stride, sel_count, sel_len, out, lse, ws, ws_bytes, stream, 0, seq_ids,
                      kv->num_seqs);
}

int sspec_unified_attn_naive(const sspec_paged_kv* kv, const uint16_t* q, const int32_t* ctx_lens,
                             const int32_t* bucket_ids, int32_t verify_bucket, int32_t num_seqs, int32_t max_verify,
                             int32_t max_ctx, int32_t num_q_heads, int32_t k, double s, float sm_scale,
                             int32_t* sel_idx, int32_t sel_stride, int32_t* sel_count, int32_t* sel_len,
                             uint16_t* out, float* lse, void* ws, size_t ws_bytes, void* stream) {
  return unified_impl(kv, q, ctx_lens, bucket_ids, verify_bucket, num_seqs, max_verify, max_ctx, num_q_heads, k, s,
                      sm_scale, sel_idx, sel_stride, sel_count, sel_len, out, lse, ws, ws_bytes, stream, 1, nullptr, 0);
}

}  // extern "C"

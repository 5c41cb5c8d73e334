/*
 * sspec.h -- C ABI of the SparseSpec attention hot path on AMD MI355X (gfx950).
 *
 * Method source: the talk-notes page "Accelerating Large-Scale Reasoning
 * Model Inference with Sparse Self-Speculative Decoding" (MLSys 2026).
 * Sections cited: "PillarAttn: dynamic sparse attention" (paper §4.1,
 * Fig. 7), "Unified batch scheduler" (paper §4.2, Fig. 8, §5.6 Fig. 15),
 * "Experimental setup" (paper §5.4: s = 0.05, k = 8).
 *
 * One decode iteration of self-speculative decoding runs, per attention
 * layer:
 *   - verify: full attention of the k+1 verification queries of a request
 *     over its whole paged KV cache, dumping every logit and each query's
 *     log-sum-exp (LSE)                                  [PillarAttn, §4.1]
 *   - PillarAttn selection: scores recovered from the dump as
 *     exp(logit - LSE), averaged over the k+1 queries and the query heads of
 *     each GQA group, Top-K (K = ceil(s*L)) per KV head  [PillarAttn, §4.1]
 *   - sparse draft attention: one draft query per request attends only to
 *     the selected tokens (plus the tokens appended since the selection)
 *                                                         [PillarAttn, §4.1]
 *   - unified: one persistent launch serving a mixed batch in which the
 *     requests of one bucket verify and all others draft
 *                                            [Unified batch scheduler, §4.2]
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers.  Every array argument is a DEVICE pointer, allocated and owned
 *   by the caller; the library never allocates or frees device memory on a
 *   call path and keeps no pointer after a call returns.  Buffers must stay
 *   alive until the stream reaches the enqueued work.  `stream` is a
 *   hipStream_t passed as void* (NULL = the default stream).
 * bfloat16.  Tensors typed `uint16_t` hold bfloat16 bit patterns.
 * Shapes.  head_dim must be 128 and page_size 16; num_q_heads must be a
 *   multiple of num_kv_heads with G = num_q_heads / num_kv_heads in
 *   {1,2,3,4,5,6,7,8}; 0 <= k <= 16 and G*(k+1) <= 128.  Query head g uses
 *   KV head g / G.
 * Paged KV.  Token j of request r lives in physical page
 *   block_table[r*bt_stride + j/16], slot j%16; the key row is
 *   k_pages[((page*num_kv_heads + h)*16 + slot)*128 + 0..127] (same for V).
 *   A request may hold at most bt_stride*16 tokens.
 * Positions.  A request with context length L (the tokens already written
 *   to its pages, the current queries included) has its k+1 verify queries
 *   at positions L-k-1 .. L-1, query i seeing keys 0 .. L-k-1+i (causal);
 *   its draft query sits at position L-1.
 * Scaling.  logit = sm_scale * dot(q, k); LSE is in natural log.
 * Workspace.  Each entry point takes a device workspace of at least
 *   sspec_*_workspace_size(...) bytes, 256-byte aligned.  Before its first
 *   use a workspace must be cleared once with sspec_workspace_init(); every
 *   call that completes leaves it ready for the next call, of any entry
 *   point and any sizes (the library clears the workspace's small
 *   zero-state region itself, with one extra fill kernel on `stream`, when
 *   the previous call on that workspace used a different layout).  Calls
 *   that share a workspace must be ordered (same stream); concurrent calls
 *   need separate ones.  After a launch that set SSPEC_DEV_ERR_WAIT_TIMEOUT
 *   the workspace holds stale state: sspec_read_device_error() reports the
 *   bit and marks the workspace for a full clear before its next use; a
 *   launch that finds stale state does nothing and sets
 *   SSPEC_DEV_ERR_WS_STATE.
 * Errors.  Every call returns an sspec_status.  Arguments are validated on
 *   the host before any HIP call; on failure nothing is launched and
 *   sspec_last_error() (thread-local) describes the problem.  Bad DATA found
 *   on the device (a context length beyond max_ctx or the block table, a
 *   physical page or selected index out of range, a verify context shorter
 *   than k+1, more verify requests than max_verify) never faults: the
 *   affected item is skipped or the entry masked, and a bit is set in the
 *   workspace's device error word, read with sspec_read_device_error().
 * Determinism.  Results do not depend on the order in which work-groups run.
 */
#ifndef SSPEC_H
#define SSPEC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SSPEC_OK = 0,
  SSPEC_ERR_INVALID_ARG = 1,  /* null pointer, negative size, bad stride ... */
  SSPEC_ERR_UNSUPPORTED = 2,  /* shape outside the supported set (see above) */
  SSPEC_ERR_WORKSPACE = 3,    /* workspace missing, too small or misaligned */
  SSPEC_ERR_HIP = 4           /* a HIP runtime call failed */
} sspec_status;

/* Bits of the device error word. */
#define SSPEC_DEV_ERR_CTX_RANGE 0x1u      /* ctx_len > max_ctx or > bt_stride*16, or < 1 */
#define SSPEC_DEV_ERR_PAGE_RANGE 0x2u     /* block-table entry outside [0, num_pages) */
#define SSPEC_DEV_ERR_SEL_RANGE 0x4u      /* selected index < 0; sel_count outside [0, sel_stride];
                                             or sel_len outside [0, max_ctx] */
#define SSPEC_DEV_ERR_VERIFY_SHORT 0x8u   /* verify ctx_len < k+1 */
#define SSPEC_DEV_ERR_TOO_MANY_VERIFY 0x10u /* unified: more verify requests than max_verify */
#define SSPEC_DEV_ERR_WAIT_TIMEOUT 0x20u  /* unified: a bounded in-kernel wait gave up */
#define SSPEC_DEV_ERR_SEQ_RANGE 0x40u     /* seq_ids entry outside [0, num_seqs) */
#define SSPEC_DEV_ERR_LAYOUT 0x80u        /* device and host disagree on the workspace layout
                                             (a mis-built library); the launch did nothing */
#define SSPEC_DEV_ERR_WS_STATE 0x100u     /* the workspace was not initialised, or holds state
                                             left by an aborted launch; the launch did nothing */

/* Paged KV cache of one attention layer (all pointers on the device). */
typedef struct sspec_paged_kv {
  const uint16_t* k_pages;     /* bf16 [num_pages][num_kv_heads][page_size][head_dim] */
  const uint16_t* v_pages;     /* same layout as k_pages */
  const int32_t* block_table;  /* [num_seqs][bt_stride]: logical page -> physical page */
  int32_t num_pages;
  int32_t num_kv_heads;
  int32_t head_dim;            /* must be 128 */
  int32_t page_size;           /* must be 16 */
  int32_t bt_stride;           /* entries per block-table row */
  int32_t num_seqs;            /* rows of block_table (requests) */
} sspec_paged_kv;

/* Thread-local description of the last non-OK status returned on this thread. */
const char* sspec_last_error(void);

/* Clear a workspace (launches one fill kernel on `stream`). */
int sspec_workspace_init(void* ws, size_t ws_bytes, void* stream);

/* Read (and with clear != 0, reset) the device error word of a workspace.
 * Synchronizes `stream`; *flags receives the SSPEC_DEV_ERR_* bits.  When
 * SSPEC_DEV_ERR_WAIT_TIMEOUT or SSPEC_DEV_ERR_WS_STATE is set the
 * workspace's zero-state region is cleared before its next use. */
int sspec_read_device_error(void* ws, int clear, void* stream, uint32_t* flags);

/* ------------------------------------------------------------------ verify
 * Full causal attention of the k+1 verify queries of n requests, with the
 * logit + LSE dump [PillarAttn, paper §4.1].
 *   q       bf16 [n][k+1][num_q_heads][128]; row i is the query at L-k-1+i
 *   seq_ids int32 [n]: request (block-table row) of item i, in [0, num_seqs)
 *   ctx_lens int32 [num_seqs]: L per request, indexed by request; each used
 *           L must satisfy k+1 <= L <= max_ctx
 *   out     bf16 [n][k+1][num_q_heads][128]
 *   lse     f32  [n][k+1][num_q_heads]
 *   logits  f32, in blocks of one page (16 keys) per KV head:
 *           [n][num_kv_heads][logit_stride/16][Mp][16], Mp = round_up(G*(k+1), 4).
 *           The logit of query i, query head g (KV head h = g / G), key j is
 *           logits[((item*num_kv_heads + h)*logit_stride + 16*(j/16))*Mp
 *                  + 16*((g % G)*(k+1) + i) + j%16]
 *           and is -inf where key j is masked for that query.  Keys in
 *           [L, round_up(L,16)) and the Mp - G*(k+1) padding rows are written
 *           -inf; blocks past round_up(L,16) are untouched.  logit_stride is a
 *           multiple of 16 in [round_up(max_ctx,16), 2^20 + 16].  (Each block
 *           is the verify kernel's accumulator layout, so every page's logits
 *           go out as contiguous 1 KB stores.)
 */
size_t sspec_verify_workspace_size(int32_t n, int32_t max_ctx, int32_t num_q_heads,
                                   int32_t num_kv_heads, int32_t k);
int sspec_verify_attn(const sspec_paged_kv* kv, const uint16_t* q, const int32_t* seq_ids,
                      const int32_t* ctx_lens, int32_t n, int32_t max_ctx,
                      int32_t num_q_heads, int32_t k, float sm_scale, uint16_t* out,
                      float* lse, float* logits, int64_t logit_stride, void* ws,
                      size_t ws_bytes, void* stream);

/* ------------------------------------------------------------- pillar_topk
 * PillarAttn selection from a verify dump [PillarAttn, paper §4.1].  For
 * item i (request r = seq_ids[i], L = ctx_lens[r]) and KV head h:
 *   S[j] = mean over the G query heads g of group h and the k+1 queries q
 *          of exp(logit(i, g, q, j) - lse[i][q][g])   (0 where masked),
 *          logit(...) read from the page-blocked layout of sspec_verify_attn
 *   K    = min(L, ceil(s * L)) evaluated in IEEE double
 *   sel_idx[r][h][0..K) = the K largest S[j], exact ties to the lower j,
 *          in ascending order of j
 *   sel_count[r] = K, sel_len[r] = L.
 *   logits/lse: as written by sspec_verify_attn (same n, k, logit_stride).
 *   sel_idx int32 [num_seqs][num_kv_heads][sel_stride], sel_stride >=
 *           ceil(s * max_ctx); only rows of the listed requests are written.
 *   0 < s <= 1.
 */
size_t sspec_pillar_topk_workspace_size(int32_t n, int32_t max_ctx, int32_t num_kv_heads);
int sspec_pillar_topk(const float* logits, const float* lse, int64_t logit_stride,
                      const int32_t* seq_ids, const int32_t* ctx_lens, int32_t n,
                      int32_t num_seqs, int32_t max_ctx, int32_t num_q_heads,
                      int32_t num_kv_heads, int32_t k, double s, int32_t* sel_idx,
                      int32_t sel_stride, int32_t* sel_count, int32_t* sel_len, void* ws,
                      size_t ws_bytes, void* stream);

/* Allocation-free variant of sspec_pillar_topk, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same arguments and results, minus
 * ws/ws_bytes.  Its workspace is a static 64 MiB device array of the library
 * (one per GPU, held until the process ends); a call whose workspace would
 * exceed it (sspec_pillar_topk_workspace_size(...) > 64 MiB) returns
 * SSPEC_ERR_WORKSPACE and launches nothing.  The first call on a GPU clears
 * the array with one fill kernel on `stream`.  Every call on one GPU shares
 * the array: calls that overlap on one GPU (other streams, other threads)
 * race and must not be issued. */
int sspec_pillar_topk_noalloc(const float* logits, const float* lse, int64_t logit_stride,
                              const int32_t* seq_ids, const int32_t* ctx_lens, int32_t n,
                              int32_t num_seqs, int32_t max_ctx, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t k, double s, int32_t* sel_idx,
                              int32_t sel_stride, int32_t* sel_count, int32_t* sel_len,
                              void* stream);

/* ----------------------------------------------------- sparse_draft_attn
 * One draft step [PillarAttn, paper §4.1]: the query of item i (request
 * r = seq_ids[i], position ctx_lens[r]-1) attends, for KV head h, to
 *   A_h = { j in sel_idx[r][h][0..sel_count[r]) : j < min(sel_len[r], L) }
 *         U [sel_len[r], L)          (tokens appended since the selection)
 * with L = ctx_lens[r].  An empty A_h gives out = 0 and lse = -inf.
 *   q   bf16 [n][num_q_heads][128];  out bf16 [n][num_q_heads][128]
 *   lse f32 [n][num_q_heads], may be NULL
 *   sel_idx/sel_count/sel_len: as written by sspec_pillar_topk (the entries
 *   of a row are distinct and ascending; a repeated index would be attended
 *   once per entry).  Selected indices at or past min(sel_len, L) are left
 *   out without an error (sspec_kv_rollback lowers sel_len below some of
 *   them); only the first min(sel_count, sel_len) entries are read.
 */
size_t sspec_draft_workspace_size(int32_t n, int32_t max_ctx, int32_t num_q_heads,
                                  int32_t num_kv_heads);
int sspec_sparse_draft_attn(const sspec_paged_kv* kv, const uint16_t* q, const int32_t* seq_ids,
                            const int32_t* ctx_lens, const int32_t* sel_idx, int32_t sel_stride,
                            const int32_t* sel_count, const int32_t* sel_len, int32_t n,
                            int32_t max_ctx, int32_t num_q_heads, float sm_scale,
                            uint16_t* out, float* lse, void* ws, size_t ws_bytes,
                            void* stream);

/* ------------------------------------------------------------ unified_attn
 * One persistent launch over all num_seqs requests of a unified batch
 * [Unified batch scheduler, paper §4.2, Fig. 8; fused kernel, §5.6 Fig. 15].
 * Request r verifies when bucket_ids[r] == verify_bucket, else it drafts.
 *   q    bf16 [rows][num_q_heads][128], rows packed in request order: k+1
 *        rows (the verify queries) for a verifying request, 1 row for a
 *        drafting one; out has the same layout; lse f32 [rows][num_q_heads].
 *   A verifying request runs sspec_verify_attn + sspec_pillar_topk
 *   semantics (its logit dump stays in the workspace) and rewrites
 *   sel_idx[r], sel_count[r] = K, sel_len[r] = ctx_lens[r].  A drafting
 *   request runs sspec_sparse_draft_attn semantics with its current
 *   sel_idx/sel_count/sel_len.
 *   num_seqs <= 512; at most max_verify requests may verify.
 */
size_t sspec_unified_workspace_size(int32_t num_seqs, int32_t max_verify, int32_t max_ctx,
                                    int32_t num_q_heads, int32_t num_kv_heads, int32_t k);
int sspec_unified_attn(const sspec_paged_kv* kv, const uint16_t* q, const int32_t* ctx_lens,
                       const int32_t* bucket_ids, int32_t verify_bucket, int32_t num_seqs,
                       int32_t max_verify, int32_t max_ctx, int32_t num_q_heads, int32_t k,
                       double s, float sm_scale, int32_t* sel_idx, int32_t sel_stride,
                       int32_t* sel_count, int32_t* sel_len, uint16_t* out, float* lse,
                       void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------- unified (naive)
 * The naive-batching baseline of the fused kernel [Unified batch scheduler,
 * paper §4.2 and §5.6 Fig. 15: one launch that serves drafts and verifies
 * with ONE tile configuration, against which the fused kernel's per-kind
 * templates are compared].  Same arguments, results and workspace as
 * sspec_unified_attn; only the drafting requests run differently: in the
 * verify's tile shape (ceil(G*(k+1)/16) MFMA query tiles, of which the one
 * draft query fills G columns and the rest is computed padding) and cut into
 * the launch's verify chunk length instead of draft-sized chunks.  Drafts
 * therefore agree with sspec_unified_attn within rounding (other chunk
 * boundaries), verifies and selections bit for bit.  G*(k+1) <= 48, else
 * SSPEC_ERR_UNSUPPORTED.  For measurement; not a faster path.
 */
int sspec_unified_attn_naive(const sspec_paged_kv* kv, const uint16_t* q, const int32_t* ctx_lens,
                             const int32_t* bucket_ids, int32_t verify_bucket, int32_t num_seqs,
                             int32_t max_verify, int32_t max_ctx, int32_t num_q_heads, int32_t k,
                             double s, float sm_scale, int32_t* sel_idx, int32_t sel_stride,
                             int32_t* sel_count, int32_t* sel_len, uint16_t* out, float* lse,
                             void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- kv_append
 * Write the current tokens' keys and values into the paged cache, before the
 * attention of the same iteration reads them [Dynamic KV-Cache management,
 * paper §4.4: each decode step adds the KV of every request's new tokens].
 * Request r (r < num_seqs) carries n_r rows: k+1 (its verify tokens) when
 * bucket_ids[r] == verify_bucket, else 1 (its draft token), packed in
 * request order like the q of sspec_unified_attn:
 *   k_new, v_new  bf16 [rows][num_kv_heads][128], rows = sum of n_r
 * Row i of request r is the token at position ctx_lens[r] - n_r + i
 * (ctx_lens as passed to sspec_unified_attn: the context including these
 * tokens); it is copied bit for bit to page block_table[r][pos/16], slot
 * pos%16 of kv->k_pages and kv->v_pages.  THIS CALL WRITES the pools the
 * struct describes (their const qualifiers serve the attention calls).
 * A row whose position is outside [0, bt_stride*16) or whose page is outside
 * [0, num_pages) is skipped; when err (a device word, may be NULL) is given,
 * SSPEC_DEV_ERR_CTX_RANGE / SSPEC_DEV_ERR_PAGE_RANGE is or-ed into it.
 * 0 <= num_seqs <= kv->num_seqs, 0 <= k <= 16; no workspace.
 */
int sspec_kv_append(const sspec_paged_kv* kv, const uint16_t* k_new, const uint16_t* v_new,
                    const int32_t* ctx_lens, const int32_t* bucket_ids, int32_t verify_bucket,
                    int32_t num_seqs, int32_t k, uint32_t* err, void* stream);

/* -------------------------------------------------------------- kv_rollback
 * After a verify, keep only the accepted tokens [Delayed verification, paper
 * §4.3: the verify phase accepts a prefix of the k drafts].  For every
 * request r < num_seqs with bucket_ids[r] == verify_bucket, with a =
 * accepted[r] clamped to [0, k]:
 *   ctx_lens[r] -= k - a       (the first verify token and a drafts remain)
 *   sel_len[r]   = min(sel_len[r], ctx_lens[r])
 * Other requests are untouched.  The rejected rows stay in the pages past
 * the context, and the next sspec_kv_append overwrites them.  All arrays are
 * device int32 [num_seqs]; runs on the device (no host synchronisation).
 */
int sspec_kv_rollback(const int32_t* bucket_ids, int32_t verify_bucket, const int32_t* accepted,
                      int32_t num_seqs, int32_t k, int32_t* ctx_lens, int32_t* sel_len,
                      void* stream);

/* ------------------------------------------------------ pack / unpack pages
 * Whole pages of the paged cache to and from one contiguous buffer [Dynamic
 * KV-Cache management, paper §4.4: a request's KV cache moves between GPU
 * and host memory in chunks].  For i < n_pages, page p = pages[i] (device
 * int32 array; host-mapped pinned memory works too):
 *   buf[(2*i + 0) * B .. +B) <-> k_pages[p * B .. +B)
 *   buf[(2*i + 1) * B .. +B) <-> v_pages[p * B .. +B),   B = num_kv_heads*16*128
 * (bf16 elements), copied bit for bit: pack reads the pools, unpack writes
 * them (THIS CALL WRITES the pools the struct describes).  A page id outside
 * [0, num_pages) is skipped and, when err (a device word, may be NULL) is
 * given, SSPEC_DEV_ERR_PAGE_RANGE is or-ed into it.  0 <= n_pages <= 65535;
 * buf and the pools 16-byte aligned; no workspace.
 */
int sspec_kv_pack_pages(const sspec_paged_kv* kv, const int32_t* pages, int32_t n_pages,
                        uint16_t* dst, uint32_t* err, void* stream);
int sspec_kv_unpack_pages(const sspec_paged_kv* kv, const int32_t* pages, int32_t n_pages,
                          const uint16_t* src, uint32_t* err, void* stream);

/* ------------------------------------------------------------ offload engine
 * Asynchronous, chunked, FIFO movement of requests' KV caches between the
 * GPU and a pinned host arena [Dynamic KV-Cache management, paper §4.4: when
 * GPU memory runs short, requests' caches are offloaded to host memory a
 * chunk at a time and loaded back later, both in FIFO order for fairness;
 * the transfers overlap the GPU's decoding].
 *
 * One engine serves one paged cache (one layer's pools).  Host-side state
 * only: the caller owns every buffer and the side stream.
 *   staging   device buffer of at least slots*chunk_pages*page_bytes bytes
 *             (page_bytes = sspec_offload_page_bytes(num_kv_heads): one
 *             page's K and V blocks), 256-byte aligned;
 *   host      pinned host memory (hipHostMalloc / torch pin_memory) of
 *             sspec_offload_host_bytes(...) bytes, 256-byte aligned: a table
 *             of page ids (read by the data movers) and room for host_pages
 *             pages of offloaded caches;
 *   side_stream  a hipStream_t of default priority on which every transfer
 *             runs (never the stream of the attention launches).
 * sspec_offload_evict(req, pages) queues a copy of the request's pages to a
 * new place in the host arena (SSPEC_ERR_WORKSPACE when the arena is full);
 * sspec_offload_restore(req, pages) queues the copy back into `pages` (the
 * same count, any physical pages; the caller writes them into the block
 * table).  Jobs run strictly in the order queued: a job's chunks are issued
 * only after every chunk of the jobs before it.  sspec_offload_pump issues
 * up to max_chunks chunks (at most `slots` in flight), each after
 * after_event (an event recorded on the attention stream, or NULL): evict =
 * pack kernel into a staging slot + device-to-host copy; restore =
 * host-to-device copy + unpack kernel.  sspec_offload_poll never blocks: it
 * retires finished chunks and reports finished jobs in FIFO order (req and
 * SSPEC_OFFLOAD_EVICT: its device pages may be reused; SSPEC_OFFLOAD_RESTORE:
 * its pages hold the cache again and its host space is free).  The caller
 * must not write an evicting request's pages, nor read a restoring one's,
 * before poll reports the job.  SSPEC_OFFLOAD_DRY: no device work at all
 * (buffers may be NULL, chunks finish at once): the planning logic alone.
 * sspec_offload_trace copies the issued chunks as int32 quadruples (req,
 * kind, first page index within the job, pages).  The engine is not
 * thread-safe; sspec_offload_destroy waits for the side stream.
 */
#define SSPEC_OFFLOAD_EVICT 1
#define SSPEC_OFFLOAD_RESTORE 2
#define SSPEC_OFFLOAD_DRY 1
typedef struct sspec_offload sspec_offload;
size_t sspec_offload_page_bytes(int32_t num_kv_heads);
size_t sspec_offload_host_bytes(int32_t num_kv_heads, int32_t chunk_pages, int32_t slots,
                                int64_t host_pages);
int sspec_offload_create(const sspec_paged_kv* kv, int32_t chunk_pages, int32_t slots, void* staging,
                         size_t staging_bytes, void* host, size_t host_bytes, void* side_stream,
                         int32_t flags, sspec_offload** out);
int sspec_offload_destroy(sspec_offload* eng);
int sspec_offload_evict(sspec_offload* eng, int32_t req, const int32_t* pages, int32_t n_pages);
int sspec_offload_restore(sspec_offload* eng, int32_t req, const int32_t* pages, int32_t n_pages);
int sspec_offload_pump(sspec_offload* eng, void* after_event, int32_t max_chunks);
int sspec_offload_poll(sspec_offload* eng, int32_t* reqs, int32_t* kinds, int32_t cap, int32_t* n_done);
int sspec_offload_pending(const sspec_offload* eng, int32_t* jobs, int32_t* chunks_in_flight,
                          int64_t* host_pages_free);
int sspec_offload_trace(const sspec_offload* eng, int32_t* out, int32_t cap, int32_t* n);

/* ------------------------------------------------ unified / append by slot
 * The same launches with the batch's requests named by slot: item i of the
 * batch (num_items items, q/out rows packed per item as in
 * sspec_unified_attn) is request slot seq_ids[i] (device int32 [num_items],
 * distinct, each in [0, kv->num_seqs)): ctx_lens, sel_idx, sel_count,
 * sel_len and the block table are indexed by slot, bucket_ids by item.  A
 * live scheduler keeps every request's state in a stable slot while the
 * batch changes from one iteration to the next [Unified batch scheduler,
 * paper §4.2].  The workspace is laid out for min(kv->num_seqs, 512) items
 * (size it with sspec_unified_workspace_size(that count, ...)), so batches
 * of different sizes share it without a re-layout.  A slot outside
 * [0, kv->num_seqs) is skipped with
 * SSPEC_DEV_ERR_SEQ_RANGE (in err for the append).  Otherwise as
 * sspec_unified_attn and sspec_kv_append.
 */
int sspec_unified_attn_slots(const sspec_paged_kv* kv, const uint16_t* q, const int32_t* seq_ids,
                             const int32_t* ctx_lens, const int32_t* bucket_ids, int32_t verify_bucket,
                             int32_t num_items, int32_t max_verify, int32_t max_ctx, int32_t num_q_heads,
                             int32_t k, double s, float sm_scale, int32_t* sel_idx, int32_t sel_stride,
                             int32_t* sel_count, int32_t* sel_len, uint16_t* out, float* lse, void* ws,
                             size_t ws_bytes, void* stream);
int sspec_kv_append_slots(const sspec_paged_kv* kv, const uint16_t* k_new, const uint16_t* v_new,
                          const int32_t* seq_ids, const int32_t* ctx_lens, const int32_t* bucket_ids,
                          int32_t verify_bucket, int32_t num_items, int32_t k, uint32_t* err, void* stream);

/* ------------------------------------------------------------------ scheduler
 * The unified batch scheduler with delayed verification [Unified batch
 * scheduler, paper §4.2, Fig. 8; Delayed verification, paper §4.3, Fig. 9].
 * Host-side integer state only (no device memory, no GPU call).
 *   admit: a new request joins the bucket with the fewest live requests
 *     (lowest id on ties) and takes the lowest free slot; its context is
 *     prompt_len (the tokens whose KV is written).
 *   next: forms iteration t (t = 0, 1, ...): verify_bucket = t mod (k+1);
 *     every live request not waiting runs, in admission order: as a verify
 *     when its bucket is the verify bucket, else as a draft; either way its
 *     context grows by one.  Outputs per item: req_ids (may be NULL),
 *     seq_ids (slots), bucket_ids; per slot (arrays of max_slots):
 *     ctx_lens (the context the attention of iteration t sees) and sel_len
 *     (the selection length the device holds, clamped after rollbacks);
 *     n_items, n_verify, verify_bucket, iter.
 *   resolve(t, accepted_by_slot): consumes iteration t's verify results
 *     (accepted drafts per slot, clamped to [0, drafts held]): the context
 *     drops by the rejected drafts, a + 1 tokens are committed, and a request
 *     whose committed output reached max_new leaves (its id is reported in
 *     `finished`, its slot and bucket place are freed).
 *   With delayed != 0, iteration t may be formed once iterations <= t-2 are
 *   resolved, and a request that verified in iteration t sits out t+1: the
 *   host reads t's results while t+1 runs.  With delayed == 0 iteration t
 *   needs t-1 resolved (the host waits for the GPU every iteration).
 *   Out-of-order calls return SSPEC_ERR_INVALID_ARG.
 * sspec_accept_stub (device, on `stream`) stands in for the model's
 * acceptance: the verify of request req_ids[i] (items with bucket_ids[i] ==
 * verify_bucket) in iteration `iter` accepts the leading drafts j = 0, 1, ...
 * (at most k) whose uniform (SplitMix64(seed ^ req << 40 ^ iter << 8 ^ j)
 * >> 11) * 2^-53 is below `rate`; the count goes to accepted_by_slot[seq_ids[i]].
 */
typedef struct sspec_sched sspec_sched;
int sspec_sched_create(int32_t k, int32_t max_slots, int32_t delayed, sspec_sched** out);
int sspec_sched_destroy(sspec_sched* sched);
int sspec_sched_admit(sspec_sched* sched, int32_t req_id, int32_t prompt_len, int32_t max_new,
                      int32_t* slot, int32_t* bucket);
int sspec_sched_next(sspec_sched* sched, int32_t* req_ids, int32_t* seq_ids, int32_t* bucket_ids,
                     int32_t* n_items, int32_t* n_verify, int32_t* verify_bucket, int64_t* iter,
                     int32_t* ctx_lens, int32_t* sel_len);
int sspec_sched_resolve(sspec_sched* sched, int64_t iter, const int32_t* accepted_by_slot,
                        int32_t* finished, int32_t cap, int32_t* n_finished);
int sspec_sched_query(const sspec_sched* sched, int32_t slot, int32_t* req_id, int32_t* ctx,
                      int32_t* out_tokens, int32_t* bucket);
int sspec_accept_stub(const int32_t* req_ids, const int32_t* seq_ids, const int32_t* bucket_ids,
                      int32_t verify_bucket, int32_t n_items, int32_t k, int64_t iter, double rate,
                      uint64_t seed, int32_t num_slots, int32_t* accepted_by_slot, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SSPEC_H */

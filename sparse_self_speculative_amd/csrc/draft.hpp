// Sparse draft attention over the critical tokens [talk notes "Accelerating
// Large-Scale Reasoning Model Inference with Sparse Self-Speculative
// Decoding", section PillarAttn, paper §4.1: the draft loads and computes
// only the critical tokens chosen at the last verify; the pattern is kept
// for the k following draft steps, paper Fig. 7].
//
// A draft task = (request, KV head, positions [p0, p1) of the token set),
// run by ONE wave.  The token set of KV head h is the selected indices still
// inside the context, followed by the tokens appended since the selection.
//   * the row ids (page * Hkv + h) * 16 + slot of kDraftSub positions at a
//     time sit in an LDS table; the next table is filled while the current
//     one is consumed (index loads hidden behind the first half, block-table
//     loads behind the second half);
//   * tiles of 16 rows (key and value) are gathered into the wave's LDS ring
//     with asynchronous global->LDS loads, two to four tiles ahead, in the
//     same swizzled layout as a verify page, and computed two at a time;
//   * each tile runs on MFMA like a verify page with one query tile: the G
//     query heads are the columns of S^T = K Q^T (the other 16 - G columns
//     are padding; MFMA issue is far cheaper than the vector-ALU dot products
//     it replaces), online softmax per column, O^T += V^T P^T with P as a
//     bf16 hi + lo pair.
#pragma once

#include "ring.hpp"
#include "verify.hpp"
#include "sspec_common.hpp"

namespace sspec {

struct DraftItem {
  const uint16_t* kp;
  const uint16_t* vp;
  const int32_t* bt;      // block-table row of the request
  int num_pages, hkv, hq, G;
  float scale;
  const uint16_t* q;      // [hq][128]
  const int32_t* sel;     // sel_idx + r*hkv*sel_stride
  int sel_stride;
  int n_sel;              // entries of sel used (clamped, see make_draft_item)
  int sel_len, L;
  int ncols;              // live query columns: G (run-time copy, naive-batching form)
  uint64_t* wait_ticks;   // task-trace builds: time spent waiting for tiles (else null)
  uint64_t* phases;       // task-trace builds: [table fill, spans, epilogue] times (else null)
  uint16_t* out;          // [hq][128]
  float* lse;             // [hq] or null
  uint32_t* err;
};

__host__ __device__ inline int draft_set_size(int n_sel, int sel_len, int L) {
  return n_sel + (L > sel_len ? L - sel_len : 0);
}

constexpr uint32_t kBadRow = 0xffffffffu;

// Per-wave LDS of a draft task: the ring and two row-id tables, then room
// that, with the second table (unused by a task of at most kDraftSub
// positions), holds the request's block-table row: kBtCache pages.
struct DraftWaveLds {
  static constexpr int kRing = 4;   // slots: three tiles in flight while one is used
  static constexpr int kTabOff = kRing * kSlotBytes;
  static constexpr int kBtExtra = 704;   // entries past the second table (the 4-wave LDS budget's rest)
  static constexpr int kBtCache = kDraftSub + kBtExtra;
  static constexpr int kBytes = kTabOff + 2 * kDraftSub * 4 + kBtExtra * 4;
};

// Token of set position `pos` for KV head h, or -1 when masked.  A selected
// index at or past min(sel_len, L) is left out without an error: a rollback
// after a verify lowers sel_len below some of the selected indices.
__device__ __forceinline__ int draft_token(const DraftItem& it, const int32_t* selrow, int pos, int p1,
                                           int lim) {
  if (pos >= p1) return -1;
  if (pos < it.n_sel) {
    const int j = selrow[pos];
    if (j < 0) set_error(it.err, SSPEC_DEV_ERR_SEL_RANGE);
    return (j >= 0 && j < lim) ? j : -1;
  }
  return it.sel_len + (pos - it.n_sel);
}

__device__ __forceinline__ uint32_t draft_row(const DraftItem& it, int h, int j) {
  if (j < 0) return kBadRow;
  int phys = it.bt[j >> 4];
  if (phys < 0 || phys >= it.num_pages) {
    set_error(it.err, SSPEC_DEV_ERR_PAGE_RANGE);
    return kBadRow;
  }
  return ((uint32_t)phys * (uint32_t)it.hkv + (uint32_t)h) * kPage + (uint32_t)(j & (kPage - 1));
}

// First half of one tile (16 gathered rows) read from its ring slot, on
// MFMA: the G query heads of the one draft query are the columns of
// S^T = K Q^T (columns G..15 are padding), the verify's tile layout with one
// query tile, so the tile's second half is the verify's (verify_page_back).
// Row 4*grp + r of the tile is key position tpos + 4*grp + r; a position past
// the span, or one whose token is not in the set, gets logit -inf and a zero
// value row (the row itself was loaded from pool row 0, which may hold
// anything, NaN included: P = 0 times it must not reach the output).
// NQ > 1 is the naive-batching form: the tile runs with the verify's NQ
// query tiles, all of whose columns past the live ones (it.ncols, a run-time
// value) are computed and masked, as a template shared by every item kind
// computes them.
template <int NQ>
__device__ __forceinline__ bool draft_tile_front(const DraftItem& it, const char* slot, const uint32_t* tab, int tpos,
                                                 int tend, const u32x4 (&qreg)[NQ][4], const VerifyState<NQ>& st,
                                                 int col, int grp, PageRegs<NQ>& pr) {
  u32x4 kr[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) kr[s] = *reinterpret_cast<const u32x4*>(slot + ring_chunk(col, 4 * s + grp));
#pragma unroll
  for (int e = 0; e < 4; ++e) pr.vr[e] = *reinterpret_cast<const u32x4*>(slot + 4096 + ring_chunk(4 * grp + e, col));
  f32x4 acc[NQ];
#pragma unroll
  for (int qt = 0; qt < NQ; ++qt) acc[qt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int qt = 0; qt < NQ; ++qt) acc[qt] = mfma16x16x32(as_bf16x8(kr[s]), as_bf16x8(qreg[qt][s]), acc[qt]);
  bool rowok[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int t = 4 * grp + r;
    rowok[r] = tpos + t < tend;   // never read past the current table
    if (rowok[r]) rowok[r] = tab[t] != kBadRow;
  }
  bool up = false;
#pragma unroll
  for (int qt = 0; qt < NQ; ++qt) {
    const bool real_col = 16 * qt + col < (NQ == 1 ? it.G : it.ncols);
#pragma unroll
    for (int r = 0; r < 4; ++r) pr.x[qt][r] = (real_col && rowok[r]) ? acc[qt][r] * it.scale : kNegInf;
    float v = fmaxf(fmaxf(pr.x[qt][0], pr.x[qt][1]), fmaxf(pr.x[qt][2], pr.x[qt][3]));
    v = max_xor16(v);
    pr.mx[qt] = max_xor32(v);
    up |= pr.mx[qt] > st.m[qt] + kRescale;
  }
  if (__ballot(!(rowok[0] && rowok[1] && rowok[2] && rowok[3])) != 0ull) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (!rowok[e]) pr.vr[e] = u32x4{0, 0, 0, 0};
  }
  return __ballot(up) != 0ull;
}

// Positions [a, b) of the current table (which starts at position q0), in
// tiles of 16 streamed through the ring (one query tile: two tiles at a
// time, two to four ahead; the naive-batching form: one at a time, R-1
// ahead).
template <int NQ>
__device__ __forceinline__ void draft_span(const DraftItem& it, const uint32_t* tab, int q0, int a, int b,
                                           char* wlds, const u32x4 (&qreg)[NQ][4], VerifyState<NQ>& st, int lane) {
  constexpr int R = NQ == 1 ? DraftWaveLds::kRing : VerifyQ<NQ>::kRing, D = R - 1;
  const int col = lane & 15, grp = lane >> 4;
  const int nk = a < b ? cdiv(b - a, 16) : 0;
  const uint32_t ring_base = lds_addr(wlds);
  auto issue = [&](int k) __attribute__((always_inline)) {
    lds_reads_done();
    const int pos = a + 16 * k;
    uint32_t rows[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int t = 4 * c + (lane >> 4);
      const uint32_t r = (pos + t < b) ? tab[pos + t - q0] : kBadRow;
      rows[c] = r == kBadRow ? 0u : r;   // masked rows read row 0; draft_tile_front zeroes them
    }
    ring_issue_rows(ring_base + (uint32_t)((k % R) * kSlotBytes), it.kp, it.vp, rows, lane);
  };
  if constexpr (NQ == 1) {
    // Two tiles at a time: both tiles' products and maxima, then both
    // halves with exponentials and P*V, so the two dependency chains overlap
    // (one wave per SIMD: each chain alone leaves the SIMD idle between
    // dependent instructions).  All R slots are filled first; the slots of
    // the pair just read take the tiles R and R+1 further on, so two to four
    // tiles are in flight.
    static_assert(R == 4, "the pair loop takes 2 of 4 slots");
#pragma unroll
    for (int j = 0; j < R; ++j)
      if (j < nk) issue(j);
    for (int k = 0; k < nk; k += 2) {
      const bool two = k + 1 < nk;
      // issued so far: tiles [0, min(nk, k + R)); tiles k (and k+1) must
      // have landed, so the loads of the later ones may stay outstanding
      const int later = min(nk, k + R) - (k + (two ? 2 : 1));
      const uint64_t tw = SSPEC_TRACE ? __builtin_amdgcn_s_memrealtime() : 0;
      if (later >= 2) wait_vm<16>();
      else if (later == 1) wait_vm<8>();
      else wait_vm<0>();
      if (SSPEC_TRACE && it.wait_ticks) *it.wait_ticks += __builtin_amdgcn_s_memrealtime() - tw;
      const int pos = a + 16 * k;
      PageRegs<1> pr0, pr1;
      draft_tile_front<1>(it, wlds + (k % R) * kSlotBytes, tab + (pos - q0), pos, b, qreg, st, col, grp, pr0);
      if (two)
        draft_tile_front<1>(it, wlds + ((k + 1) % R) * kSlotBytes, tab + (pos + 16 - q0), pos + 16, b, qreg, st, col,
                            grp, pr1);
      if (k + R < nk) issue(k + R);           // into the slot of tile k, read above
      if (k + R + 1 < nk) issue(k + R + 1);   // into the slot of tile k+1
      if (__ballot(pr0.mx[0] > st.m[0] + kRescale) != 0ull) verify_rescale<1>(st, pr0);
      verify_page_back<1>(st, pr0);
      if (two) {
        if (__ballot(pr1.mx[0] > st.m[0] + kRescale) != 0ull) verify_rescale<1>(st, pr1);
        verify_page_back<1>(st, pr1);
      }
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < D; ++j)
    if (j < nk) issue(j);
  for (int k = 0; k < nk; ++k) {
    // tiles k+1 .. k+D-1 are the only later memory operations
    const uint64_t tw = SSPEC_TRACE ? __builtin_amdgcn_s_memrealtime() : 0;
    if (k + D - 1 < nk) wait_vm<8 * (D - 1)>();
    else wait_vm_dyn(8 * max(0, nk - 1 - k));
    if (SSPEC_TRACE && it.wait_ticks) *it.wait_ticks += __builtin_amdgcn_s_memrealtime() - tw;
    if (k + D < nk) issue(k + D);    // into the slot of tile k-1
    const int pos = a + 16 * k;
    PageRegs<NQ> pr;
    if (draft_tile_front<NQ>(it, wlds + (k % R) * kSlotBytes, tab + (pos - q0), pos, b, qreg, st, col, grp, pr))
      verify_rescale<NQ>(st, pr);
    verify_page_back<NQ>(st, pr);
  }
}

// Attention of one draft query over set positions [p0, p1) of KV head h, by
// the calling wave.  `part` null: write the final O/LSE; otherwise write the
// split partial (part_split_bytes(G): O rows in accumulator unit order, then
// (m, l) per row) with coherent stores.  NQ: query
// tiles of the MFMA tile shape (1; more only in the naive-batching form,
// where tile 0 holds the G live columns and the rest is padding).
template <int G, int NQ = 1>
__device__ SSPEC_TASK void draft_wave_range(const DraftItem& it, int h, int p0, int p1, float* part, char* wlds) {
  const int lane = (int)lane_id();
  const uint64_t ph0 = SSPEC_TRACE ? __builtin_amdgcn_s_memrealtime() : 0;
  const int lim = min(it.sel_len, it.L);
  const int32_t* selrow = it.sel + (int64_t)h * it.sel_stride;
  uint32_t* tabs = reinterpret_cast<uint32_t*>(wlds + DraftWaveLds::kTabOff);   // [2][kDraftSub]
  constexpr int kPer = kDraftSub / kWave;

  // Q^T operands: lane (col, grp) holds query head col (< G), dims
  // 32*s + 8*grp .. +7 of k-step s
  const int col = lane & 15, grp = lane >> 4;
  u32x4 qreg[NQ][4];
#pragma unroll
  for (int qt = 0; qt < NQ; ++qt) {
    const int c = 16 * qt + col;
    const bool live = c < (NQ == 1 ? G : it.ncols);
#pragma unroll
    for (int s = 0; s < 4; ++s)
      qreg[qt][s] = live ? *reinterpret_cast<const u32x4*>(it.q + (int64_t)(h * G + c) * kD + 32 * s + 8 * grp)
                         : u32x4{0, 0, 0, 0};
  }
  VerifyState<NQ> st;
#pragma unroll
  for (int qt = 0; qt < NQ; ++qt) {
    st.m[qt] = kNegInf;
    st.l[qt] = 0.f;
#pragma unroll
    for (int n = 0; n < 8; ++n) st.o[qt][n] = f32x4{0.f, 0.f, 0.f, 0.f};
    st.lim[qt] = 0;
  }

  // first table (a wave's LDS writes are seen by its later LDS reads).  A
  // task of one table over a context of at most kBtCache pages loads the
  // request's block-table row into LDS together with the selected indices,
  // so its row ids take one round trip rather than two dependent ones.
  const int npg_ctx = cdiv(it.L, kPage);   // every token of the set is < L
  if (p1 - p0 <= kDraftSub && npg_ctx <= DraftWaveLds::kBtCache) {
    constexpr int kBtPer = (DraftWaveLds::kBtCache + kWave - 1) / kWave;
    int32_t* btc = reinterpret_cast<int32_t*>(tabs + kDraftSub);
    int bv[kBtPer];
#pragma unroll
    for (int t = 0; t < kBtPer; ++t) {
      const int idx = lane + kWave * t;
      bv[t] = idx < npg_ctx ? it.bt[idx] : 0;
    }
    int j[kPer];
#pragma unroll
    for (int e = 0; e < kPer; ++e) j[e] = draft_token(it, selrow, p0 + lane + kWave * e, p1, lim);
#pragma unroll
    for (int t = 0; t < kBtPer; ++t) {
      const int idx = lane + kWave * t;
      if (idx < npg_ctx) btc[idx] = bv[t];
    }
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      uint32_t row = kBadRow;
      if (j[e] >= 0) {
        const int phys = btc[j[e] >> 4];
        if (phys < 0 || phys >= it.num_pages) set_error(it.err, SSPEC_DEV_ERR_PAGE_RANGE);
        else row = ((uint32_t)phys * (uint32_t)it.hkv + (uint32_t)h) * kPage + (uint32_t)(j[e] & (kPage - 1));
      }
      tabs[lane + kWave * e] = row;
    }
  } else {
    int j[kPer];
#pragma unroll
    for (int e = 0; e < kPer; ++e) j[e] = draft_token(it, selrow, p0 + lane + kWave * e, p1, lim);
#pragma unroll
    for (int e = 0; e < kPer; ++e) tabs[lane + kWave * e] = draft_row(it, h, j[e]);
  }
  uint64_t ph1 = 0;
  if (SSPEC_TRACE && it.phases) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    ph1 = __builtin_amdgcn_s_memrealtime();
    it.phases[0] += ph1 - ph0;
  }
  const int nsub = cdiv(p1 - p0, kDraftSub);
  for (int sub = 0; sub < nsub; ++sub) {
    const uint32_t* tab = tabs + (sub & 1) * kDraftSub;
    uint32_t* ntab = tabs + ((sub + 1) & 1) * kDraftSub;
    const int q0 = p0 + sub * kDraftSub;
    const int q1 = min(q0 + kDraftSub, p1);
    const bool more = sub + 1 < nsub;
    // with a next table to fill, split the positions in two spans so its
    // loads hide behind them; otherwise stream all in one span
    const int half = more ? min(q0 + round_up(cdiv(q1 - q0, 2), 16), q1) : q1;
    int j[kPer];
    if (more) {
#pragma unroll
      for (int e = 0; e < kPer; ++e) j[e] = draft_token(it, selrow, q1 + lane + kWave * e, p1, lim);
    }
    draft_span<NQ>(it, tab, q0, q0, half, wlds, qreg, st, lane);
    uint32_t nrow[kPer];
    if (more) {
#pragma unroll
      for (int e = 0; e < kPer; ++e) nrow[e] = draft_row(it, h, j[e]);
    }
    draft_span<NQ>(it, tab, q0, half, q1, wlds, qreg, st, lane);
    if (more) {
#pragma unroll
      for (int e = 0; e < kPer; ++e) ntab[lane + kWave * e] = nrow[e];
    }
  }

  uint64_t ph2 = 0;
  if (SSPEC_TRACE && it.phases) {
    ph2 = __builtin_amdgcn_s_memrealtime();
    it.phases[1] += ph2 - ph1;
  }
  // the 4 lane groups of a column hold partial sums of l; O^T is complete:
  // lane (col, grp) holds head col, dims 8*(4*grp + r) + n in st.o[0][n][r]
  st.l[0] = sum_xor32(sum_xor16(st.l[0]));
  if (col < G) {
    if (part == nullptr) {
      const float ls = st.l[0];
      const float inv = ls > 0.f ? 1.f / ls : 0.f;
      uint16_t* orow = it.out + (int64_t)(h * G + col) * kD;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v[8];
#pragma unroll
        for (int n = 0; n < 8; ++n) v[n] = st.o[0][n][r];
        store_out_row8(orow + 8 * (4 * grp + r), v, inv);
      }
      if (grp == 0 && it.lse) it.lse[h * G + col] = ls > 0.f ? st.m[0] + __logf(ls) : kNegInf;
    } else {
      // unit 4*(2r + nh) + grp holds dims 32*grp + 8*r + 4*nh .. +3
      float* prow = part + (int64_t)col * kD + 4 * grp;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        st_coh4(prow + 32 * r, f32x4{st.o[0][0][r], st.o[0][1][r], st.o[0][2][r], st.o[0][3][r]});
        st_coh4(prow + 32 * r + 16, f32x4{st.o[0][4][r], st.o[0][5][r], st.o[0][6][r], st.o[0][7][r]});
      }
      if (grp == 0) st_coh4(part + G * kD + 4 * col, f32x4{st.m[0], st.l[0], 0.f, 0.f});
    }
  }
  if (SSPEC_TRACE && it.phases) {
    drain_vm();
    it.phases[2] += __builtin_amdgcn_s_memrealtime() - ph2;
  }
}

// Merge the draft split partials (nsplit of part_split_bytes(G)) of one (item, KV head) with
// coherent loads, four heads at a time: lane l takes head g0 + l/16, dims
// 8*(l%16) .. +7.  The splits are merged in index order with a running
// maximum (fixed order: the result does not depend on which wave merges);
// the loads of 8 splits are in flight together.
template <int G>
__device__ SSPEC_TASK void draft_wave_combine(const DraftItem& it, int h, const float* parts, int nsplit) {
  const int lane = (int)lane_id();
  parts = wave_uniform(parts);
  const uint32_t split_bytes = part_split_bytes(G);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(parts, (uint32_t)nsplit * split_bytes);
  const int d8 = (lane & 15) * 8;
  // dims d8 .. d8+3 and d8+4 .. d8+7 sit in units part_unit(d8) and part_unit(d8) + 4
  const uint32_t unit = (uint32_t)part_unit(d8) * 16u;
#pragma unroll
  for (int g0 = 0; g0 < G; g0 += 4) {
    const int g = g0 + (lane >> 4);
    const int gl = min(g, G - 1);
    float mx = kNegInf, ls = 0.f;
    f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < nsplit; s0 += 8) {
      f32x4 o0[8], o1[8];
      float ms[8], lv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        // splits past the end read 0 from outside the range and are skipped
        const uint32_t b = (uint32_t)(s0 + u) * split_bytes;
        o0[u] = ld_coh4(rs, b + (uint32_t)(gl * kD * 4) + unit);
        o1[u] = ld_coh4(rs, b + (uint32_t)(gl * kD * 4) + unit + 64u);
        const uint32_t ml = b + (uint32_t)((G * kD + 4 * gl) * 4);
        ms[u] = ld_coh1(rs, ml);
        lv[u] = ld_coh1(rs, ml + 4u);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (s0 + u >= nsplit) break;
        const float mn = fmaxf(mx, ms[u]);
        if (mn == kNegInf) continue;   // nothing visible so far
        const float fo = fast_exp2((mx - mn) * kLog2e), fn = fast_exp2((ms[u] - mn) * kLog2e);
        ls = ls * fo + lv[u] * fn;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          a0[c] = a0[c] * fo + o0[u][c] * fn;
          a1[c] = a1[c] * fo + o1[u][c] * fn;
        }
        mx = mn;
      }
    }
    if (g < G) {
      const float inv = ls > 0.f ? 1.f / ls : 0.f;
      float v[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
      store_out_row8(it.out + (int64_t)(h * G + g) * kD + d8, v, inv);
      if ((lane & 15) == 0 && it.lse) it.lse[h * G + g] = ls > 0.f ? mx + __logf(ls) : kNegInf;
    }
  }
}

}  // namespace sspec

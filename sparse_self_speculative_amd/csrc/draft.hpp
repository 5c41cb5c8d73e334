// Sparse draft attention over the critical tokens [talk notes "Accelerating
// Large-Scale Reasoning Model Inference with Sparse Self-Speculative
// Decoding", section PillarAttn, paper §4.1: the draft loads and computes
// only the critical tokens chosen at the last verify; the pattern is kept
// for the k following draft steps, paper Fig. 7].
//
// A draft task = (request, KV head, positions [p0, p1) of the token set),
// run by ONE wave.  The token set of KV head h is the selected indices still
// inside the context, followed by the tokens appended since the selection.
// This is a gather of 256-byte key/value rows, far below the MFMA ridge, so
// it runs on the vector ALU:
//   * the row ids (page * Hkv + h) * 16 + slot of kDraftSub positions at a
//     time sit in an LDS table; the next table is filled while the current
//     one is consumed (index loads hidden behind the first half, block-table
//     loads behind the second half);
//   * tiles of 16 rows (key and value) are gathered into the wave's LDS ring
//     with asynchronous global->LDS loads, three tiles ahead;
//   * 8 lanes share one row (16 dims = 32 bytes each); the G query-head dot
//     products use bf16 dot2 and a 3-step DPP reduction inside each 8-lane
//     half-row, and P*V uses bf16 dot2 over the lane's two rows (P as a bf16
//     hi + lo pair, so it keeps fp32-like precision); every lane group keeps
//     its own online-softmax state, merged once at the end (DPP row rotate
//     by 8, v_permlane16/32_swap).
#pragma once

#include "ring.hpp"
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
  uint16_t* out;          // [hq][128]
  float* lse;             // [hq] or null
  uint32_t* err;
};

__host__ __device__ inline int draft_set_size(int n_sel, int sel_len, int L) {
  return n_sel + (L > sel_len ? L - sel_len : 0);
}

constexpr uint32_t kBadRow = 0xffffffffu;

// Per-wave LDS of a draft task: the ring and two row-id tables.
struct DraftWaveLds {
  static constexpr int kRing = 4;   // slots: three tiles in flight while one is used
  static constexpr int kTabOff = kRing * kSlotBytes;
  static constexpr int kBytes = kTabOff + 2 * kDraftSub * 4;
};

// Token of set position `pos` for KV head h, or -1 when masked.
__device__ __forceinline__ int draft_token(const DraftItem& it, const int32_t* selrow, int pos, int p1,
                                           int lim) {
  if (pos >= p1) return -1;
  if (pos < it.n_sel) {
    const int j = selrow[pos];
    if (j < 0 || j >= it.sel_len) set_error(it.err, SSPEC_DEV_ERR_SEL_RANGE);
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

// sum over the 8 lanes of each DPP half-row
__device__ __forceinline__ float row8_sum(float x) {
  x += SSPEC_DPP(x, 0xB1);   // quad_perm [1,0,3,2]
  x += SSPEC_DPP(x, 0x4E);   // quad_perm [2,3,0,1]
  x += SSPEC_DPP(x, 0x141);  // row_half_mirror
  return x;
}

// One tile (16 gathered rows) read from its ring slot.  Lane
// (rg8 = l/8, q8 = l%8) works on rows rg8 and rg8 + 8, dims 16*q8 .. +15.
template <int G>
__device__ __forceinline__ void draft_tile(const DraftItem& it, const char* slot, const uint32_t* tab, int tpos,
                                           int tend, const uint32_t (&qv)[G][8], float (&m)[G], float (&l)[G],
                                           float (&o)[G][16], int lane) {
  const int rg8 = lane >> 3, q8 = lane & 7;
  u32x4 k[2][2], v[2][2];
  bool ok[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int t = rg8 + 8 * e;
    uint32_t rid = kBadRow;
    if (tpos + t < tend) rid = tab[t];   // never read past the current table
    ok[e] = rid != kBadRow;
    k[e][0] = *reinterpret_cast<const u32x4*>(slot + ring_chunk(t, 2 * q8));
    k[e][1] = *reinterpret_cast<const u32x4*>(slot + ring_chunk(t, 2 * q8 + 1));
    v[e][0] = *reinterpret_cast<const u32x4*>(slot + 4096 + ring_chunk(t, 2 * q8));
    v[e][1] = *reinterpret_cast<const u32x4*>(slot + 4096 + ring_chunk(t, 2 * q8 + 1));
    if (!ok[e]) v[e][0] = v[e][1] = u32x4{0, 0, 0, 0};
  }
  float x[2][G];
#pragma unroll
  for (int e = 0; e < 2; ++e)
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float d = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) d = dot2_bf16(qv[g][i], k[e][0][i], d);
#pragma unroll
      for (int i = 0; i < 4; ++i) d = dot2_bf16(qv[g][4 + i], k[e][1][i], d);
      d = row8_sum(d);
      x[e][g] = ok[e] ? d * it.scale : kNegInf;
    }
  // value pairs (row rg8, row rg8 + 8) of each of the lane's 16 dims
  uint32_t vp[16];
#pragma unroll
  for (int c = 0; c < 16; ++c) vp[c] = sel_half(v[0][c >> 3][(c >> 1) & 3], v[1][c >> 3][(c >> 1) & 3], c & 1);
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float mx = fmaxf(x[0][g], x[1][g]);
    if (mx > m[g] + kRescale) {   // lazy rescale (see kRescale)
      if (m[g] != kNegInf) {
        const float alpha = fast_exp2((m[g] - mx) * kLog2e);
        l[g] *= alpha;
#pragma unroll
        for (int c = 0; c < 16; ++c) o[g][c] *= alpha;
      }
      m[g] = mx;
    }
    if (m[g] == kNegInf) continue;
    const float mb = m[g] * kLog2e;
    const float p0 = fast_exp2(x[0][g] * kLog2e - mb), p1 = fast_exp2(x[1][g] * kLog2e - mb);
    l[g] += p0 + p1;
    uint32_t ph, pl;   // bf16 hi + lo pair of (p0, p1), see split_bf2
    split_bf2(p0, p1, ph, pl);
#pragma unroll
    for (int c = 0; c < 16; ++c) o[g][c] = dot2_bf16(pl, vp[c], dot2_bf16(ph, vp[c], o[g][c]));
  }
}

// Positions [a, b) of the current table (which starts at position q0), in
// tiles of 16 streamed through the ring three tiles ahead.
template <int G>
__device__ __forceinline__ void draft_span(const DraftItem& it, const uint32_t* tab, int q0, int a, int b,
                                           char* wlds, const uint32_t (&qv)[G][8], float (&m)[G], float (&l)[G],
                                           float (&o)[G][16], int lane) {
  constexpr int R = DraftWaveLds::kRing, D = R - 1;
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
      rows[c] = r == kBadRow ? 0u : r;   // masked rows read row 0 and are discarded
    }
    ring_issue_rows(ring_base + (uint32_t)((k % R) * kSlotBytes), it.kp, it.vp, rows, lane);
  };
#pragma unroll
  for (int j = 0; j < D; ++j)
    if (j < nk) issue(j);
  for (int k = 0; k < nk; ++k) {
    // tiles k+1 .. k+D-1 are the only later memory operations
    if (k + D - 1 < nk) wait_vm<8 * (D - 1)>();
    else wait_vm_dyn(8 * max(0, nk - 1 - k));
    if (k + D < nk) issue(k + D);    // into the slot of tile k-1
    const int pos = a + 16 * k;
    draft_tile<G>(it, wlds + (k % R) * kSlotBytes, tab + (pos - q0), pos, b, qv, m, l, o, lane);
  }
}

// Attention of one draft query over set positions [p0, p1) of KV head h, by
// the calling wave.  `part` null: write the final O/LSE; otherwise write the
// partial [G][kPartStride] (o[128], m, l) with coherent stores.
template <int G>
__device__ SSPEC_TASK void draft_wave_range(const DraftItem& it, int h, int p0, int p1, float* part, char* wlds) {
  const int lane = (int)lane_id();
  const int q8 = lane & 7;
  const int lim = min(it.sel_len, it.L);
  const int32_t* selrow = it.sel + (int64_t)h * it.sel_stride;
  uint32_t* tabs = reinterpret_cast<uint32_t*>(wlds + DraftWaveLds::kTabOff);   // [2][kDraftSub]
  constexpr int kPer = kDraftSub / kWave;

  uint32_t qv[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const u32x4* src = reinterpret_cast<const u32x4*>(it.q + (int64_t)(h * G + g) * kD + 16 * q8);
    const u32x4 a = src[0], b = src[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      qv[g][i] = a[i];
      qv[g][4 + i] = b[i];
    }
  }
  float m[G], l[G], o[G][16];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = kNegInf;
    l[g] = 0.f;
#pragma unroll
    for (int c = 0; c < 16; ++c) o[g][c] = 0.f;
  }

  // first table (a wave's LDS writes are seen by its later LDS reads)
  {
    int j[kPer];
#pragma unroll
    for (int e = 0; e < kPer; ++e) j[e] = draft_token(it, selrow, p0 + lane + kWave * e, p1, lim);
#pragma unroll
    for (int e = 0; e < kPer; ++e) tabs[lane + kWave * e] = draft_row(it, h, j[e]);
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
    draft_span<G>(it, tab, q0, q0, half, wlds, qv, m, l, o, lane);
    uint32_t nrow[kPer];
    if (more) {
#pragma unroll
      for (int e = 0; e < kPer; ++e) nrow[e] = draft_row(it, h, j[e]);
    }
    draft_span<G>(it, tab, q0, half, q1, wlds, qv, m, l, o, lane);
    if (more) {
#pragma unroll
      for (int e = 0; e < kPer; ++e) ntab[lane + kWave * e] = nrow[e];
    }
  }

  // merge the 8 lane groups (lanes 8, 16 and 32 apart share dims)
#pragma unroll
  for (int g = 0; g < G; ++g) {
    // row_ror:8 pairs lane i with lane i^8 of its 16-lane row: same dims,
    // neighbouring row group
    const float m8 = fmaxf(m[g], SSPEC_DPP(m[g], 0x128));
    const float mw = max_xor32(max_xor16(m8));
    const float f = (mw == kNegInf) ? 0.f : fast_exp2((m[g] - mw) * kLog2e);
    float lv = l[g] * f;
    lv += SSPEC_DPP(lv, 0x128);
    l[g] = sum_xor32(sum_xor16(lv));
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      float v = o[g][c] * f;
      v += SSPEC_DPP(v, 0x128);
      o[g][c] = sum_xor32(sum_xor16(v));
    }
    m[g] = mw;
  }
  // lanes 0..7 (row group 0) now hold the whole state; lane q8 owns dims
  // 16*q8 .. +15
  if (lane < 8) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if (part == nullptr) {
        const float inv = l[g] > 0.f ? 1.f / l[g] : 0.f;
        uint16_t* orow = it.out + (int64_t)(h * G + g) * kD + 16 * q8;
        float v0[8], v1[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          v0[c] = o[g][c];
          v1[c] = o[g][8 + c];
        }
        uint4 a, b;
        a.x = pack_bf2(v0[0] * inv, v0[1] * inv);
        a.y = pack_bf2(v0[2] * inv, v0[3] * inv);
        a.z = pack_bf2(v0[4] * inv, v0[5] * inv);
        a.w = pack_bf2(v0[6] * inv, v0[7] * inv);
        b.x = pack_bf2(v1[0] * inv, v1[1] * inv);
        b.y = pack_bf2(v1[2] * inv, v1[3] * inv);
        b.z = pack_bf2(v1[4] * inv, v1[5] * inv);
        b.w = pack_bf2(v1[6] * inv, v1[7] * inv);
        reinterpret_cast<uint4*>(orow)[0] = a;
        reinterpret_cast<uint4*>(orow)[1] = b;
        if (q8 == 0 && it.lse) it.lse[h * G + g] = l[g] > 0.f ? m[g] + __logf(l[g]) : kNegInf;
      } else {
        float* prow = part + (int64_t)g * kPartStride;
#pragma unroll
        for (int c = 0; c < 16; c += 4)
          st_coh4(prow + 16 * q8 + c, f32x4{o[g][c], o[g][c + 1], o[g][c + 2], o[g][c + 3]});
        if (q8 == 0) {
          st_coh(prow + kD, m[g]);
          st_coh(prow + kD + 1, l[g]);
        }
      }
    }
  }
}

// Merge draft partials [nsplit][G][kPartStride] of one (item, KV head) with
// coherent loads; lane l handles dims 2l, 2l+1.
template <int G>
__device__ SSPEC_TASK void draft_wave_combine(const DraftItem& it, int h, const float* parts, int nsplit) {
  const int lane = (int)lane_id();
#pragma unroll 1
  for (int g = 0; g < G; ++g) {
    float ms = kNegInf;
    for (int s = 0; s < nsplit; ++s) ms = fmaxf(ms, ld_coh(parts + ((int64_t)s * G + g) * kPartStride + kD));
    float ls = 0.f, a0 = 0.f, a1 = 0.f;
    if (ms != kNegInf) {
      for (int s = 0; s < nsplit; ++s) {
        const float* pr = parts + ((int64_t)s * G + g) * kPartStride;
        const float f = fast_exp2((ld_coh(pr + kD) - ms) * kLog2e);
        ls += ld_coh(pr + kD + 1) * f;
        a0 += ld_coh(pr + 2 * lane) * f;
        a1 += ld_coh(pr + 2 * lane + 1) * f;
      }
    }
    const float inv = ls > 0.f ? 1.f / ls : 0.f;
    *reinterpret_cast<uint32_t*>(it.out + (int64_t)(h * G + g) * kD + 2 * lane) = pack_bf2(a0 * inv, a1 * inv);
    if (lane == 0 && it.lse) it.lse[h * G + g] = ls > 0.f ? ms + __logf(ls) : kNegInf;
  }
}

}  // namespace sspec

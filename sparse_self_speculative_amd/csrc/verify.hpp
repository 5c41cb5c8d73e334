// Verify attention with the logit + LSE dump [talk notes "Accelerating
// Large-Scale Reasoning Model Inference with Sparse Self-Speculative
// Decoding", section PillarAttn, paper §4.1: the verify kernel emits the
// attention scores as logits and log-sum-exp while it computes full
// attention].
//
// One task = (request, KV head, chunk of cp pages), run by ONE wave.
// The G query heads of the KV head's group times the k+1 verify queries form
// M = G*(k+1) rows, padded to NQT tiles of 16.  The chunk's page table sits
// in the wave's LDS, the Q^T operands in registers (more than 4 tiles: an
// LDS copy of the Q tile).  Per page (16 keys) the wave does:
//   S^T = K * Q^T   on 16x16x32 bf16 MFMA (K page = A operand, Q^T = B);
//   scale, causal mask, store the logits (fp32, 16 B per lane);
//   softmax per query column against a reference fixed for the pass over
//                   the chunk (column maxima across the 4 lane groups with
//                   v_permlane16/32_swap; a second pass if logits climb far
//                   above it, see verify_wave_chunk);
//   O^T += V^T * P^T  on 16x16x16 MFMA: P^T comes out of the S^T accumulator
//                   layout unchanged (as a bf16 hi + lo pair); V^T is built in
//                   registers by assigning O^T row i of d-tile n to
//                   d = 8*i + n, so no transpose is needed.
// Pages stream through the wave's LDS ring (ring.hpp), three pages ahead (two
// with more than 3 query tiles).
// A multi-chunk context leaves one partial per chunk; the wave that
// finishes the last chunk merges them (verify_wave_lse, verify_wave_out).
#pragma once

#include "ring.hpp"
#include "sspec_common.hpp"

namespace sspec {

struct VerifyItem {
  const uint16_t* kp;
  const uint16_t* vp;
  const int32_t* bt;    // block-table row of the request
  int num_pages, hkv, hq, kp1, G, M;
  int L;                // context length
  float scale;
  const uint16_t* q;    // query row i, head g at q + i*q_row_stride + g*128
  int64_t q_row_stride;
  float* dump;          // page-blocked logits of the item: (KV head h, key j, row m) at
                        // dump + (h*lstride + 16*(j/16))*mp + 16*m + j%16,
                        // row m = gi*kp1 + i
  int64_t lstride;      // keys per KV head in the dump (multiple of 16)
  int mp;               // rows per page block: round_up(M, 4)
  uint16_t* out;        // query row i, head g at out + i*out_row_stride + g*128
  int64_t out_row_stride;
  float* lse;           // query row i, head g at lse + i*lse_row_stride + g
  int64_t lse_row_stride;
  uint32_t* err;
};

// Up to 3 query tiles the Q^T operands stay in registers for the whole
// chunk (16 VGPRs per tile); more tiles read them from an LDS copy of the Q
// tile at every page.  With the operands in LDS, each QK^T product waited on
// its own LDS read; in registers the tiles' products issue back to back.
template <int NQT>
struct VerifyQ {
  static constexpr bool kRegs = NQT <= 3;
  // ring slots: the LDS the Q tile leaves free holds a fourth slot, so three
  // pages are in flight while one is computed
  static constexpr int kRing = kRegs ? 4 : 3;
};

// Per-wave LDS of a verify task: the ring, the chunk's page table and (more
// than 4 query tiles) the Q tile, bf16 rows padded to 272 B so the 16-byte
// operand reads are free of bank conflicts.
template <int NQT>
struct VerifyWaveLds {
  static constexpr int kQStride = kD + 8;
  static constexpr int kPages = kVChunkMax;
  static constexpr int kPagesOff = VerifyQ<NQT>::kRing * kSlotBytes;
  static constexpr int kQOff = kPagesOff + kPages * 4;
  static constexpr int kBytes = kQOff + (VerifyQ<NQT>::kRegs ? 0 : NQT * 16 * kQStride * 2);
};

template <int NQT>
struct VerifyState {
  float m[NQT], l[NQT];
  f32x4 o[NQT][8];   // O^T tiles: d-tile n, lane holds query col, d = 8*(4*grp + r) + n
  int lim[NQT];      // last key index visible to this lane's query column
};

// Registers one page carries from its first half (products, logits,
// maxima) to its second (exponentials, P*V).
template <int NQT>
struct PageRegs {
  u32x4 vr[4];
  f32x4 x[NQT];
  float mx[NQT];
};

// First half of one page (16 keys, keys tb..tb+15), read from its ring slot:
// S^T = K Q^T, mask, logit dump, column maxima.  Returns whether any
// column's maximum exceeds its reference by more than kVerifyRange
// (wave-wide vote).  The dump keeps each page's logits as one contiguous block
// [mp rows][16 keys], which is the S^T accumulator layout itself: every one
// of the NQT stores writes 1 KB of consecutive bytes (the memory system takes
// these far better than scattered 64-byte row pieces).  FULL: the caller
// knows that every key of the page is visible to every query (no causal
// mask, no keys past the context), and the page runs without those tests.
template <int NQT, bool FULL = false>
__device__ __forceinline__ bool verify_page_front(const VerifyItem& it, __amdgpu_buffer_rsrc_t dump_rs, int tb,
                                                  const char* slot, const uint16_t* s_q,
                                                  const u32x4 (&qreg)[NQT][4], const VerifyState<NQT>& st,
                                                  int col, int grp, PageRegs<NQT>& pr) {
  constexpr int QS = VerifyWaveLds<NQT>::kQStride;
  u32x4 kr[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) kr[s] = *reinterpret_cast<const u32x4*>(slot + ring_chunk(col, 4 * s + grp));
#pragma unroll
  for (int e = 0; e < 4; ++e) pr.vr[e] = *reinterpret_cast<const u32x4*>(slot + 4096 + ring_chunk(4 * grp + e, col));
  if (!FULL && tb + kPage > it.L) {
    // keys past the context (tail of the last page): zero V so 0*garbage
    // cannot make NaN; their logits are masked below
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (tb + 4 * grp + e >= it.L) pr.vr[e] = u32x4{0, 0, 0, 0};
  }
  f32x4 acc[NQT];
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt) acc[qt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) {
      const u32x4 qv = VerifyQ<NQT>::kRegs ? qreg[qt][s]
                                           : *reinterpret_cast<const u32x4*>(s_q + (16 * qt + col) * QS + 32 * s + 8 * grp);
      acc[qt] = mfma16x16x32(as_bf16x8(kr[s]), as_bf16x8(qv), acc[qt]);
    }
  const bool full = FULL || tb + kPage <= it.L - it.kp1;   // every key visible to every query (wave-uniform)
  const int t0 = tb + 4 * grp;
  bool need = false;
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt) {
    f32x4& x = pr.x[qt];
    if (full) {
      // padding rows (lim -1) get -inf through the additive bias
      const float bias = st.lim[qt] >= 0 ? 0.f : kNegInf;
#pragma unroll
      for (int r = 0; r < 4; ++r) x[r] = fmaf(acc[qt][r], it.scale, bias);
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) x[r] = (t0 + r <= st.lim[qt]) ? acc[qt][r] * it.scale : kNegInf;
    }
    // rows mp.. of the last tile lie outside the block: their offset is past
    // the resource, so the store writes nothing for them (one instruction per
    // tile either way)
    const int m = 16 * qt + col;
    const uint32_t off = m < it.mp ? (uint32_t)((tb * it.mp + 16 * m + 4 * grp) * 4) : 0xfffffff0u;
    st_coh4_buf(dump_rs, off, x);
    float v = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    v = max_xor16(v);
    pr.mx[qt] = max_xor32(v);
    need |= pr.mx[qt] > st.m[qt] + kVerifyRange;
  }
  return __ballot(need) != 0ull;
}

// Lazy rescale (the draft's running softmax): the reference max only moves
// when the running max exceeds it by more than kRescale, so
// exp(x - m) <= e^kRescale stays small and the accumulators are rescaled only
// on those rare steps.  The verify instead fixes its reference per pass.
template <int NQT>
__device__ __forceinline__ void verify_rescale(VerifyState<NQT>& st, const PageRegs<NQT>& pr) {
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt) {
    const bool up = pr.mx[qt] > st.m[qt] + kRescale;
    const float alpha = (up && st.m[qt] != kNegInf) ? fast_exp2((st.m[qt] - pr.mx[qt]) * kLog2e) : 1.f;
    st.l[qt] *= alpha;
#pragma unroll
    for (int n = 0; n < 8; ++n) scale_acc(st.o[qt][n], alpha);
    st.m[qt] = up ? pr.mx[qt] : st.m[qt];
  }
}

// Second half of a page: P = exp(x - m), O^T += V^T P^T.  P enters the
// product as a bf16 hi + lo pair: a single bf16 P would add up to 2^-9
// relative error per weight, which together with the bf16 rounding of O can
// exceed 1e-2 on outputs of magnitude ~2.  Both halves go through ONE 16x16x32
// MFMA per output tile: the k index is only summed over, so lane group g's
// eight k-slots carry keys 4g..4g+3 twice -- the hi parts of P against V, then
// the lo parts against the same V (the lane already holds exactly these
// keys in the S^T accumulator layout) -- which halves the P*V instructions
// and leaves no dependent MFMA pairs.  A row whose reference is still -inf
// (a padding row) has only -inf logits: exp2(-inf - 0) = 0.
template <int NQT>
__device__ __forceinline__ void verify_page_back(VerifyState<NQT>& st, const PageRegs<NQT>& pr) {
  uint32_t p01[NQT], p23[NQT], l01[NQT], l23[NQT];
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt) {
    const float mb = st.m[qt] != kNegInf ? st.m[qt] * kLog2e : 0.f;
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) p[r] = fast_exp2(fmaf(pr.x[qt][r], kLog2e, -mb));
    st.l[qt] += (p[0] + p[1]) + (p[2] + p[3]);
    split_bf2(p[0], p[1], p01[qt], l01[qt]);
    split_bf2(p[2], p[3], p23[qt], l23[qt]);
  }
  bf16x8 pb[NQT];   // B operand: P^T of keys 4g..4g+3, hi then lo
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt) pb[qt] = as_bf16x8(u32x4{p01[qt], p23[qt], l01[qt], l23[qt]});
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    const int w = n >> 1, odd = n & 1;
    const uint32_t a0 = sel_half(pr.vr[0][w], pr.vr[1][w], odd);
    const uint32_t a1 = sel_half(pr.vr[2][w], pr.vr[3][w], odd);
    const bf16x8 va = as_bf16x8(u32x4{a0, a1, a0, a1});   // A operand: V^T of the same keys, twice
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) st.o[qt][n] = mfma16x16x32(va, pb[qt], st.o[qt][n]);
  }
}

__device__ __forceinline__ void store_out_row8(uint16_t* dst, const float (&v)[8], float inv) {
  uint4 pk;
  pk.x = pack_bf2(v[0] * inv, v[1] * inv);
  pk.y = pack_bf2(v[2] * inv, v[3] * inv);
  pk.z = pack_bf2(v[4] * inv, v[5] * inv);
  pk.w = pack_bf2(v[6] * inv, v[7] * inv);
  *reinterpret_cast<uint4*>(dst) = pk;
}

// Chunk `split` (pages [split*cp, split*cp + cp)) of one (item, KV head) by
// the calling wave.  `part` null: the chunk is the whole context, write O and
// LSE; otherwise write the split partial (part_split_bytes(M): O rows in
// accumulator unit order, then (m, l) per row) with
// coherent stores.
template <int NQT>
__device__ SSPEC_TASK void verify_wave_chunk(const VerifyItem& it, int h, int split, int cp, float* part,
                                             char* wlds) {
  using Lds = VerifyWaveLds<NQT>;
  constexpr int QS = Lds::kQStride;
  const int lane = (int)lane_id();
  const int col = lane & 15, grp = lane >> 4;
  const int M = it.M, kp1 = it.kp1;
  const int pg0 = split * cp;   // pages [pg0, pg0 + npg), cp <= kVChunkMax
  const int npg = min(cdiv(it.L, kPage) - pg0, cp);

  int* s_pages = reinterpret_cast<int*>(wlds + Lds::kPagesOff);
  uint16_t* s_q = reinterpret_cast<uint16_t*>(wlds + Lds::kQOff);
  for (int i = lane; i < npg; i += kWave) {
    int phys = it.bt[pg0 + i];
    if (phys < 0 || phys >= it.num_pages) {
      set_error(it.err, SSPEC_DEV_ERR_PAGE_RANGE);
      phys = 0;
    }
    s_pages[i] = phys;
  }
  // Q^T operands: lane (col, grp) of tile qt, k-step s holds row 16*qt + col,
  // dims 32*s + 8*grp .. +7
  u32x4 qreg[NQT][4];
  if constexpr (VerifyQ<NQT>::kRegs) {
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) {
      const int row = 16 * qt + col;
      const int gi = row / kp1, i = row - gi * kp1;
      const uint16_t* src = it.q + (int64_t)i * it.q_row_stride + (int64_t)(h * it.G + gi) * kD + 8 * grp;
#pragma unroll
      for (int s = 0; s < 4; ++s)
        qreg[qt][s] = row < M ? *reinterpret_cast<const u32x4*>(src + 32 * s) : u32x4{0, 0, 0, 0};
    }
    // take the values here, before the ring's loads are issued: a first use
    // after them would make the compiler wait for those loads as well
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt)
#pragma unroll
      for (int s = 0; s < 4; ++s) asm volatile("" : "+v"(qreg[qt][s]));
  } else {
    for (int c = lane; c < NQT * 16 * 16; c += kWave) {
      const int row = c >> 4, d8 = (c & 15) * 8;
      u32x4 v = {0, 0, 0, 0};
      if (row < M) {
        const int gi = row / kp1, i = row - gi * kp1;
        v = *reinterpret_cast<const u32x4*>(it.q + (int64_t)i * it.q_row_stride + (int64_t)(h * it.G + gi) * kD + d8);
      }
      *reinterpret_cast<u32x4*>(s_q + row * QS + d8) = v;
    }
  }

  VerifyState<NQT> st;
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt) {
    const int m = 16 * qt + col;
    st.lim[qt] = (m < M) ? it.L - kp1 + (m % kp1) : -1;
  }

  // pages stream through the R-slot ring: page k+D (D = R-1) goes into the
  // slot of page k-1 as soon as page k has landed, so pages k+1 .. k+D are in
  // flight while page k is computed
  constexpr int R = VerifyQ<NQT>::kRing, D = R - 1;
  const uint32_t ring_base = lds_addr(wlds);
  uint32_t soff[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) soff[c] = ring_src_off(c, lane);
  const size_t head_off = (size_t)h * kPage * kD;
  const size_t page_stride = (size_t)it.hkv * kPage * kD;
  auto issue = [&](int k) __attribute__((always_inline)) {
    lds_reads_done();
    const int phys = __builtin_amdgcn_readfirstlane(s_pages[k]);
    const size_t off = (size_t)phys * page_stride + head_off;
    ring_issue_page(ring_base + (uint32_t)((k % R) * kSlotBytes), it.kp + off, it.vp + off, soff);
  };
  // this (item, KV head)'s dump block: lstride*mp floats, < 2^32 bytes
  const __amdgpu_buffer_rsrc_t dump_rs =
      make_rsrc(wave_uniform(it.dump + (int64_t)h * it.lstride * it.mp), (uint32_t)(it.lstride * it.mp * 4));
  // Softmax reference per column, fixed for the whole pass: the larger of the
  // column's maximum over the chunk's first page and the floor `ref0` (kept
  // from an earlier pass).  exp(x - ref) <= e^kVerifyRange keeps P, l and O
  // far inside fp32 and bf16 range, and the accumulators are only ever
  // touched by MFMAs (any other update of O inside the page loop made the
  // compiler copy every accumulator register on every page).  If any page's
  // logits climb more than kVerifyRange above the reference, the pass runs
  // to its end (its O and l are then discarded; they may overflow) and the
  // chunk is computed once more with the reference set to the largest logit
  // of each column over the whole chunk, which no page can exceed (the dump
  // is rewritten with the same values).  So there are at most two passes.
  float ref0[NQT];
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt) ref0[qt] = kNegInf;
  for (;;) {
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) {
      st.m[qt] = ref0[qt];
      st.l[qt] = 0.f;
#pragma unroll
      for (int n = 0; n < 8; ++n) st.o[qt][n] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int j = 0; j < D; ++j)
      if (j < npg) issue(j);
    PageRegs<NQT> pr;
    bool again = false;
    float seen[NQT];
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) seen[qt] = kNegInf;
    // Any page, with every test made at run time.
    auto page = [&](int k) __attribute__((always_inline)) {
      // issued after page k: pages k+1 .. k+D-1 (8 loads each) and the NQT
      // logit stores of each of the pages k-D .. k-1 computed meanwhile;
      // waves retire memory operations in order
      if (k >= D && k + D - 1 < npg) wait_vm<8 * (D - 1) + NQT * D>();   // the steady state
      else wait_vm_dyn(8 * max(0, min(D - 1, npg - 1 - k)) + NQT * min(k, D));
      if (k + D < npg) issue(k + D);   // into the slot of page k-1
      const bool up = verify_page_front<NQT>(it, dump_rs, (pg0 + k) * kPage, wlds + (k % R) * kSlotBytes, s_q,
                                             qreg, st, col, grp, pr);
      if (k == 0) {
        // the reference; a column with no visible key yet (padding) keeps
        // -inf, and its exponentials are 0
#pragma unroll
        for (int qt = 0; qt < NQT; ++qt) st.m[qt] = fmaxf(st.m[qt], pr.mx[qt]);
      } else {
        again |= up;
      }
#pragma unroll
      for (int qt = 0; qt < NQT; ++qt) seen[qt] = fmaxf(seen[qt], pr.mx[qt]);
      verify_page_back<NQT>(st, pr);
    };
    // Pages [kA0, kA1) are the steady state -- the wait count is constant,
    // the page D ahead always exists, every key is visible to every query --
    // and run as one straight-line block with none of those tests (with one
    // wave per SIMD, every branch bubble in the page loop is lost time).
    const int kfull = min(npg, max(0, (it.L - kp1) / kPage - pg0));   // pages with tb + 16 <= L - k - 1
    const int kA0 = min(D, npg), kA1 = max(kA0, min(npg - D, kfull));
    for (int k = 0; k < kA0; ++k) page(k);
    for (int k = kA0; k < kA1; ++k) {
      wait_vm<8 * (D - 1) + NQT * D>();
      issue(k + D);
      again |= verify_page_front<NQT, true>(it, dump_rs, (pg0 + k) * kPage, wlds + (k % R) * kSlotBytes, s_q, qreg,
                                            st, col, grp, pr);
#pragma unroll
      for (int qt = 0; qt < NQT; ++qt) seen[qt] = fmaxf(seen[qt], pr.mx[qt]);
      verify_page_back<NQT>(st, pr);
    }
    for (int k = kA1; k < npg; ++k) page(k);
    if (!again) break;
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) ref0[qt] = seen[qt];
    wait_vm<0>();   // drain the ring and the stores before the pass restarts
  }

  // the 4 lane groups of a column hold partial sums of l; O^T is complete
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt) {
    st.l[qt] = sum_xor32(sum_xor16(st.l[qt]));
    const int m = 16 * qt + col;
    if (m >= M) continue;
    if (part == nullptr) {
      const float ls = st.l[qt];
      const float inv = ls > 0.f ? 1.f / ls : 0.f;
      const int gi = m / kp1, i = m - gi * kp1, g = h * it.G + gi;
      uint16_t* orow = it.out + (int64_t)i * it.out_row_stride + (int64_t)g * kD;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v[8];
#pragma unroll
        for (int n = 0; n < 8; ++n) v[n] = st.o[qt][n][r];
        store_out_row8(orow + 8 * (4 * grp + r), v, inv);
      }
      if (grp == 0) st_coh(it.lse + (int64_t)i * it.lse_row_stride + g, ls > 0.f ? st.m[qt] + __logf(ls) : kNegInf);
    } else {
      // unit 4*(2r + nh) + grp holds dims 32*grp + 8*r + 4*nh .. +3
      float* prow = part + (int64_t)m * kD + 4 * grp;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        st_coh4(prow + 32 * r, f32x4{st.o[qt][0][r], st.o[qt][1][r], st.o[qt][2][r], st.o[qt][3][r]});
        st_coh4(prow + 32 * r + 16, f32x4{st.o[qt][4][r], st.o[qt][5][r], st.o[qt][6][r], st.o[qt][7][r]});
      }
      if (grp == 0) st_coh4(part + (int64_t)M * kD + 4 * m, f32x4{st.m[qt], st.l[qt], 0.f, 0.f});
    }
  }
}

// Merging the split partials (nsplit of part_split_bytes(M)) of one (item, KV head) is
// split in two so that the selection does not wait for the output merge:
//   verify_wave_lse    LSE of every row from the (m, l) of the splits (a few
//                      KB of loads); publishes nothing itself;
//   verify_wave_out    O = sum over splits of o_s * exp(m_s - LSE).
// Both use device-coherent loads and sum the splits in a fixed order, so the
// result does not depend on which wave merges.
__device__ SSPEC_TASK void verify_wave_lse(const VerifyItem& it, int h, const float* parts, int nsplit) {
  const int lane = (int)lane_id();
  const int M = it.M, kp1 = it.kp1;
  parts = wave_uniform(parts);
  const uint32_t split_bytes = part_split_bytes(M);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(parts, (uint32_t)nsplit * split_bytes);
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int m = lane + 64 * e;   // this lane's row
    if (m >= M) continue;
    const uint32_t row = (uint32_t)((M * kD + 4 * m) * 4);   // (m, l)
    float mx = kNegInf, ls = 0.f;
    for (int s0 = 0; s0 < nsplit; s0 += 8) {
      f32x4 ml[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) ml[u] = ld_coh4(rs, (uint32_t)(s0 + u) * split_bytes + row);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (s0 + u >= nsplit || ml[u][0] == kNegInf) continue;
        const float nm = fmaxf(mx, ml[u][0]);
        ls = (mx == kNegInf ? 0.f : ls * fast_exp2((mx - nm) * kLog2e)) + ml[u][1] * fast_exp2((ml[u][0] - nm) * kLog2e);
        mx = nm;
      }
    }
    const int gi = m / kp1, i = m - gi * kp1, g = h * it.G + gi;
    st_coh(it.lse + (int64_t)i * it.lse_row_stride + g, ls > 0.f ? mx + __logf(ls) : kNegInf);
  }
}

// Rows [m0, m0 + 2*RH) of the output merge: lane half `half` takes rows
// m0 + 2r + half (r < RH), 4 dims each, SB splits of each row's loads in
// flight together (RH * SB = 32 loads of 16 bytes per lane).
template <int RH, int SB>
__device__ __forceinline__ void verify_out_rows(const VerifyItem& it, int h, __amdgpu_buffer_rsrc_t rs, uint32_t split_bytes,
                                                int nsplit, const float (&lse_r)[2], int m0, int half, int d4) {
  const int M = it.M, kp1 = it.kp1;
  int mr[RH];
  float lse[RH];
#pragma unroll
  for (int e = 0; e < RH; ++e) {
    mr[e] = min(m0 + 2 * e + half, M - 1);
    const float l0 = __shfl(lse_r[0], mr[e] & 63), l1 = __shfl(lse_r[1], mr[e] & 63);
    lse[e] = mr[e] < 64 ? l0 : l1;
  }
  f32x4 acc[RH];
#pragma unroll
  for (int e = 0; e < RH; ++e) acc[e] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int M4 = M * kD * 4;   // the (m, l) block
  const uint32_t unit = (uint32_t)part_unit(d4) * 16u;
  for (int s0 = 0; s0 < nsplit; s0 += SB) {
    f32x4 o[RH][SB];
    float ms[RH][SB];
#pragma unroll
    for (int e = 0; e < RH; ++e) {
#pragma unroll
      for (int u = 0; u < SB; ++u) {
        const uint32_t b = (uint32_t)(s0 + u) * split_bytes;
        o[e][u] = ld_coh4(rs, b + (uint32_t)(mr[e] * kD * 4) + unit);
        ms[e][u] = ld_coh1(rs, b + (uint32_t)(M4 + 16 * mr[e]));
      }
    }
#pragma unroll
    for (int e = 0; e < RH; ++e) {
#pragma unroll
      for (int u = 0; u < SB; ++u) {
        // splits past the end read 0 from outside the range: weight 0
        const float wgt = (s0 + u < nsplit && ms[e][u] != kNegInf && lse[e] != kNegInf)
                              ? fast_exp2((ms[e][u] - lse[e]) * kLog2e)
                              : 0.f;
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[e][c] += wgt * o[e][u][c];
      }
    }
  }
#pragma unroll
  for (int e = 0; e < RH; ++e) {
    const int m = m0 + 2 * e + half;
    if (m >= M) continue;
    const int gi = m / kp1, i = m - gi * kp1, g = h * it.G + gi;
    uint2 pk;
    pk.x = pack_bf2(acc[e][0], acc[e][1]);
    pk.y = pack_bf2(acc[e][2], acc[e][3]);
    *reinterpret_cast<uint2*>(it.out + (int64_t)i * it.out_row_stride + (int64_t)g * kD + d4) = pk;
  }
}

// Needs this item's LSE (written by verify_wave_lse, read back coherently).
// Each round trip merges 2*RH rows over SB splits at a time, RH * SB = 32:
// few splits take many rows per round (a pair of 4 splits and 36 rows needs
// 3 round trips, not 9).
__device__ SSPEC_TASK void verify_wave_out(const VerifyItem& it, int h, const float* parts, int nsplit) {
  const int lane = (int)lane_id();
  const int M = it.M;
  const int half = lane >> 5, d4 = (lane & 31) * 4;
  parts = wave_uniform(parts);
  const uint32_t split_bytes = part_split_bytes(M);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(parts, (uint32_t)nsplit * split_bytes);
  drain_vm();   // this wave's LSE stores are complete before they are read back
  // the LSE of rows lane and lane + 64, fetched once
  float lse_r[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int m = min(lane + 64 * e, M - 1);
    const int gi = m / it.kp1, i = m - gi * it.kp1;
    lse_r[e] = ld_coh(it.lse + (int64_t)i * it.lse_row_stride + h * it.G + gi);
  }
  if (nsplit <= 4) {
    for (int m0 = 0; m0 < M; m0 += 16) verify_out_rows<8, 4>(it, h, rs, split_bytes, nsplit, lse_r, m0, half, d4);
  } else if (nsplit <= 8) {
    for (int m0 = 0; m0 < M; m0 += 8) verify_out_rows<4, 8>(it, h, rs, split_bytes, nsplit, lse_r, m0, half, d4);
  } else {
    for (int m0 = 0; m0 < M; m0 += 4) verify_out_rows<2, 16>(it, h, rs, split_bytes, nsplit, lse_r, m0, half, d4);
  }
}

}  // namespace sspec

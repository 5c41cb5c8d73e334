// Verify attention with the logit + LSE dump [talk notes "Accelerating
// Large-Scale Reasoning Model Inference with Sparse Self-Speculative
// Decoding", section PillarAttn, paper §4.1: the verify kernel emits the
// attention scores as logits and log-sum-exp while it computes full
// attention].
//
// One task = (request, KV head, chunk of keys).  The G query heads of the
// KV head's group times the k+1 verify queries form M = G*(k+1) rows, padded
// to NQT tiles of 16.  The chunk's page table and the Q tile sit in LDS.  Per
// page (16 keys) a wave does:
//   S^T = K * Q^T   on 16x16x32 bf16 MFMA: the key page (row-major, 256 B
//                   per token) is the A operand straight from global memory,
//                   Q^T the B operand read from LDS;
//   scale, causal mask, store the logits (fp32, 16 B per lane);
//   online softmax per query column (max across the 4 lane groups with
//                   v_permlane16/32_swap);
//   O^T += V^T * P^T  on 16x16x16 MFMA: P^T comes out of the S^T accumulator
//                   layout unchanged; V^T is built in registers from 16-byte
//                   row loads by assigning O^T row i of d-tile n to
//                   d = 8*i + n, so no LDS transpose is needed.
// The 4 waves take pages round-robin, each keeping the next page's loads in
// flight while it computes the current one, and merge their (max, sum, O)
// states through LDS at the end of the chunk.
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
  const uint16_t* q;    // [kp1][hq][128] of this item
  int64_t q_row_stride; // elements between query rows i (hq*128 normally)
  float* dump;          // row (g, i) at dump + (g*kp1 + i)*lstride
  int64_t lstride;
  uint16_t* out;        // query row i, head g at out + i*out_row_stride + g*128
  int64_t out_row_stride;
  float* lse;           // query row i, head g at lse + i*lse_row_stride + g
  int64_t lse_row_stride;
  uint32_t* err;
};

// LDS of verify_chunk.  While streaming: each wave's ring of kRing tiles,
// the chunk's page table and the Q tile (bf16, rows padded to 272 B so the
// 16-byte operand reads are free of bank conflicts).  At the end: the merge
// buffers (they reuse the space).
template <int NQT>
struct VerifyLds {
  static constexpr int kQStride = kD + 8;                 // bf16 per Q row
  static constexpr int kMaxPages = kMaxCtx / 64 / kPage;  // pages of the longest chunk
  static constexpr int kObufStride = kD + 4;
  static constexpr int kRingBytes = kWaves * kRing * kSlotBytes;
  static constexpr int kPagesOff = kRingBytes;
  static constexpr int kQOff = kPagesOff + kMaxPages * 4;
  static constexpr int kLoopBytes = kQOff + NQT * 16 * kQStride * 2;
  static constexpr int kMergeBytes = (NQT * 16 * kObufStride + 2 * kWaves * NQT * 16 + 2 * NQT * 16) * 4;
  static constexpr int kBytes = kLoopBytes > kMergeBytes ? kLoopBytes : kMergeBytes;
};

template <int NQT>
struct VerifyState {
  float m[NQT], l[NQT];
  f32x4 o[NQT][8];   // O^T tiles: d-tile n, lane holds query col, d = 8*(4*grp + r) + n
  int lim[NQT];      // last key index visible to this lane's query column
};

// One page (16 keys, keys tb..tb+15) of one wave, read from its ring slot:
// S^T = K Q^T, mask, dump (exactly NQT stores), online softmax, O^T += V^T P^T.
template <int NQT>
__device__ __forceinline__ void verify_page(const VerifyItem& it, int h, int tb, const char* slot,
                                            const uint16_t* s_q, VerifyState<NQT>& st, int col, int grp) {
  constexpr int QS = VerifyLds<NQT>::kQStride;
  u32x4 kr[4], vr[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) kr[s] = *reinterpret_cast<const u32x4*>(slot + ring_chunk(col, 4 * s + grp));
#pragma unroll
  for (int e = 0; e < 4; ++e) vr[e] = *reinterpret_cast<const u32x4*>(slot + 4096 + ring_chunk(4 * grp + e, col));
  if (tb + kPage > it.L) {
    // keys past the context (tail of the last page): zero V so 0*garbage
    // cannot make NaN; their logits are masked below
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (tb + 4 * grp + e >= it.L) vr[e] = u32x4{0, 0, 0, 0};
  }
  f32x4 x[NQT];
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt) {
    f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const u32x4 qv = *reinterpret_cast<const u32x4*>(s_q + (16 * qt + col) * QS + 32 * s + 8 * grp);
      a = mfma16x16x32(as_bf16x8(kr[s]), as_bf16x8(qv), a);
    }
    const int t0 = tb + 4 * grp;
#pragma unroll
    for (int r = 0; r < 4; ++r) x[qt][r] = (t0 + r <= st.lim[qt]) ? a[r] * it.scale : kNegInf;
    // rows m >= M of the last tile are padding; lane col = 0 always holds a
    // real row (M > 16*(NQT-1)), so every wave issues exactly NQT stores
    const int m = 16 * qt + col;
    if (m < it.M) store16(it.dump + (int64_t)(h * it.M + m) * it.lstride + t0, x[qt]);
  }
  // P enters the P*V product as a bf16 hi + lo pair (two MFMAs): a single
  // bf16 P would add up to 2^-9 relative error per weight, which together
  // with the bf16 rounding of O can exceed 1e-2 on outputs of magnitude ~2
  uint32_t p01[NQT], p23[NQT], l01[NQT], l23[NQT];
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt) {
    float mx = fmaxf(fmaxf(x[qt][0], x[qt][1]), fmaxf(x[qt][2], x[qt][3]));
    mx = max_xor16(mx);
    mx = max_xor32(mx);
    // lazy rescale: the reference max only moves when the running max
    // exceeds it by more than kRescale, so exp(x - m) <= e^kRescale stays
    // small and the accumulators are rescaled only on those rare steps
    if (mx > st.m[qt] + kRescale) {
      if (st.m[qt] != kNegInf) {
        const float alpha = fast_exp2((st.m[qt] - mx) * kLog2e);
        st.l[qt] *= alpha;
#pragma unroll
        for (int n = 0; n < 8; ++n) st.o[qt][n] *= alpha;
      }
      st.m[qt] = mx;
    }
    float p[4] = {0.f, 0.f, 0.f, 0.f};
    if (st.m[qt] != kNegInf) {
      const float mb = st.m[qt] * kLog2e;
#pragma unroll
      for (int r = 0; r < 4; ++r) p[r] = fast_exp2(x[qt][r] * kLog2e - mb);
      st.l[qt] += (p[0] + p[1]) + (p[2] + p[3]);
    }
    split_bf2(p[0], p[1], p01[qt], l01[qt]);
    split_bf2(p[2], p[3], p23[qt], l23[qt]);
  }
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    const int w = n >> 1, odd = n & 1;
    const uint32_t a0 = sel_half(vr[0][w], vr[1][w], odd);
    const uint32_t a1 = sel_half(vr[2][w], vr[3][w], odd);
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) {
      st.o[qt][n] = mfma16x16x16(a0, a1, p01[qt], p23[qt], st.o[qt][n]);
      st.o[qt][n] = mfma16x16x16(a0, a1, l01[qt], l23[qt], st.o[qt][n]);
    }
  }
}

// Writes the chunk's merged state: if `part` is null the final O/LSE (the
// chunk is the whole context), otherwise the partial [M][m, l, o[128]].
template <int NQT>
__device__ void verify_chunk(const VerifyItem& it, int h, int split, float* part, char* lds_raw) {
  constexpr int QS = VerifyLds<NQT>::kQStride;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int M = it.M, kp1 = it.kp1;
  const int cl = verify_chunk_len(it.L);
  const int t0 = split * cl;
  const int t1 = min(t0 + cl, it.L);
  const int pg0 = t0 / kPage;
  const int npg = cdiv(t1, kPage) - pg0;

  int* s_pages = reinterpret_cast<int*>(lds_raw + VerifyLds<NQT>::kPagesOff);
  uint16_t* s_q = reinterpret_cast<uint16_t*>(lds_raw + VerifyLds<NQT>::kQOff);
  for (int i = threadIdx.x; i < npg; i += kThreads) {
    int phys = it.bt[pg0 + i];
    if (phys < 0 || phys >= it.num_pages) {
      set_error(it.err, SSPEC_DEV_ERR_PAGE_RANGE);
      phys = 0;
    }
    s_pages[i] = phys;
  }
  for (int c = threadIdx.x; c < NQT * 16 * 16; c += kThreads) {
    const int row = c >> 4, d8 = (c & 15) * 8;
    u32x4 v = {0, 0, 0, 0};
    if (row < M) {
      const int gi = row / kp1, i = row - gi * kp1;
      v = *reinterpret_cast<const u32x4*>(it.q + (int64_t)i * it.q_row_stride + (int64_t)(h * it.G + gi) * kD + d8);
    }
    *reinterpret_cast<u32x4*>(s_q + row * QS + d8) = v;
  }

  VerifyState<NQT> st;
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt) {
    st.m[qt] = kNegInf;
    st.l[qt] = 0.f;
#pragma unroll
    for (int n = 0; n < 8; ++n) st.o[qt][n] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int m = 16 * qt + col;
    st.lim[qt] = (m < M) ? it.L - kp1 + (m % kp1) : -1;
  }
  __syncthreads();

  // wave w streams pages w, w+4, ... (its tiles k = 0, 1, ...) through its
  // ring; tiles k+1 and k+2 are in flight while tile k is computed
  const int nk = npg > wave ? cdiv(npg - wave, kWaves) : 0;
  char* ring = lds_raw + wave * kRing * kSlotBytes;
  const uint32_t ring_base = lds_addr(ring);
  uint32_t soff[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) soff[c] = ring_src_off(c, lane);
  const size_t head_off = (size_t)h * kPage * kD;
  const size_t page_stride = (size_t)it.hkv * kPage * kD;
  auto issue = [&](int k) {
    const int phys = __builtin_amdgcn_readfirstlane(s_pages[wave + kWaves * k]);
    const size_t off = (size_t)phys * page_stride + head_off;
    ring_issue_page(ring_base + (uint32_t)((k % kRing) * kSlotBytes), it.kp + off, it.vp + off, soff);
  };
  if (nk > 0) issue(0);
  if (nk > 1) issue(1);
  for (int k = 0; k < nk; ++k) {
    // issued after tile k: tile k+1 (8 loads) and the NQT logit stores of
    // tile k-1
    wait_vm_dyn(8 * (k + 1 < nk) + NQT * (k >= 1));
    verify_page<NQT>(it, h, (pg0 + wave + kWaves * k) * kPage, ring + (k % kRing) * kSlotBytes, s_q, st, col, grp);
    if (k + 2 < nk) issue(k + 2);
  }
  __syncthreads();   // LDS is reused for the merge below

  // ---- merge the 4 waves' states through LDS
  constexpr int OS = VerifyLds<NQT>::kObufStride;
  float* obuf = reinterpret_cast<float*>(lds_raw);    // [NQT*16][OS]
  float* mw = obuf + NQT * 16 * OS;                   // [kWaves][NQT*16]
  float* lw = mw + kWaves * NQT * 16;                 // [kWaves][NQT*16]
  float* mst = lw + kWaves * NQT * 16;                // [NQT*16]
  float* lst = mst + NQT * 16;                        // [NQT*16]
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt) {
    float l = st.l[qt];
    l = sum_xor16(l);
    l = sum_xor32(l);
    if (grp == 0) {
      mw[wave * NQT * 16 + 16 * qt + col] = st.m[qt];
      lw[wave * NQT * 16 + 16 * qt + col] = l;
    }
  }
  __syncthreads();
  if (threadIdx.x < NQT * 16) {
    const int row = threadIdx.x;
    float ms = kNegInf;
    for (int w = 0; w < kWaves; ++w) ms = fmaxf(ms, mw[w * NQT * 16 + row]);
    float ls = 0.f;
    if (ms != kNegInf)
      for (int w = 0; w < kWaves; ++w)
        ls += lw[w * NQT * 16 + row] * fast_exp2((mw[w * NQT * 16 + row] - ms) * kLog2e);
    mst[row] = ms;
    lst[row] = ls;
  }
  __syncthreads();
  for (int w = 0; w < kWaves; ++w) {
    if (wave == w) {
#pragma unroll
      for (int qt = 0; qt < NQT; ++qt) {
        const int row = 16 * qt + col;
        const float ms = mst[row];
        const float f = (ms == kNegInf) ? 0.f : fast_exp2((st.m[qt] - ms) * kLog2e);
#pragma unroll
        for (int n = 0; n < 8; ++n)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int d = 8 * (4 * grp + r) + n;
            const float v = st.o[qt][n][r] * f;
            if (w == 0) obuf[row * OS + d] = v;
            else obuf[row * OS + d] += v;
          }
      }
    }
    __syncthreads();
  }

  // ---- write the final rows or the partial
  for (int idx = threadIdx.x; idx < M * (kD / 4); idx += kThreads) {
    const int m = idx / (kD / 4), d4 = (idx % (kD / 4)) * 4;
    const float* src = obuf + m * OS + d4;
    if (part == nullptr) {
      const float ls = lst[m];
      const float inv = ls > 0.f ? 1.f / ls : 0.f;
      const int gi = m / kp1, i2 = m - gi * kp1, g = h * it.G + gi;
      uint2 pk;
      pk.x = pack_bf2(src[0] * inv, src[1] * inv);
      pk.y = pack_bf2(src[2] * inv, src[3] * inv);
      *reinterpret_cast<uint2*>(it.out + (int64_t)i2 * it.out_row_stride + (int64_t)g * kD + d4) = pk;
      if (d4 == 0) it.lse[(int64_t)i2 * it.lse_row_stride + g] = ls > 0.f ? mst[m] + __logf(ls) : kNegInf;
    } else {
      float* dst = part + (int64_t)m * kPartStride;
      if (d4 == 0) {
        dst[0] = mst[m];
        dst[1] = lst[m];
      }
      dst[2 + d4 + 0] = src[0];
      dst[2 + d4 + 1] = src[1];
      dst[2 + d4 + 2] = src[2];
      dst[2 + d4 + 3] = src[3];
    }
  }
}

// Merge the partials of all splits of one (item, KV head) into O and LSE.
// parts: [nsplit][M][kPartStride]; summed in split order (deterministic).
__device__ inline void verify_combine(const VerifyItem& it, int h, const float* parts, int nsplit) {
  const int M = it.M, kp1 = it.kp1;
  for (int idx = threadIdx.x; idx < M * (kD / 4); idx += kThreads) {
    const int m = idx / (kD / 4), d4 = (idx % (kD / 4)) * 4;
    float ms = kNegInf;
    for (int s = 0; s < nsplit; ++s) ms = fmaxf(ms, parts[((int64_t)s * M + m) * kPartStride]);
    float ls = 0.f, acc[4] = {0.f, 0.f, 0.f, 0.f};
    if (ms != kNegInf) {
      for (int s = 0; s < nsplit; ++s) {
        const float* p = parts + ((int64_t)s * M + m) * kPartStride;
        const float f = fast_exp2((p[0] - ms) * kLog2e);
        ls += p[1] * f;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] += p[2 + d4 + e] * f;
      }
    }
    const float inv = ls > 0.f ? 1.f / ls : 0.f;
    const int gi = m / kp1, i = m - gi * kp1, g = h * it.G + gi;
    uint2 pk;
    pk.x = pack_bf2(acc[0] * inv, acc[1] * inv);
    pk.y = pack_bf2(acc[2] * inv, acc[3] * inv);
    *reinterpret_cast<uint2*>(it.out + (int64_t)i * it.out_row_stride + (int64_t)g * kD + d4) = pk;
    if (d4 == 0) it.lse[(int64_t)i * it.lse_row_stride + g] = ls > 0.f ? ms + __logf(ls) : kNegInf;
  }
}

}  // namespace sspec

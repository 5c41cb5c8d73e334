// Sparse draft attention over the critical tokens [talk notes "Accelerating
// Large-Scale Reasoning Model Inference with Sparse Self-Speculative
// Decoding", section PillarAttn, paper §4.1: the draft loads and computes
// only the critical tokens chosen at the last verify; the pattern is kept
// for the k following draft steps, paper Fig. 7].
//
// One task = (request, KV head, chunk of the token set).  The token set of
// KV head h is the selected indices still inside the context, followed by
// the tokens appended since the selection.  This is a gather of 256-byte
// key/value rows, far below the MFMA ridge, so it runs on the vector ALU:
// 16 lanes share one row (8 dims = 16 bytes each, 4 rows per load
// instruction), the G query-head dot products use bf16 dot2 and a 4-step
// reduction inside each 16-lane row, and every lane group keeps its own
// online-softmax state that is merged only at the end of the task.
#pragma once

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
  int n_sel;              // entries of sel used (sel_count clamped to sel_stride)
  int sel_len, L;
  uint16_t* out;          // [hq][128]
  float* lse;             // [hq] or null
  uint32_t* err;
};

__host__ __device__ inline int draft_set_size(int n_sel, int sel_len, int L) {
  return n_sel + (L > sel_len ? L - sel_len : 0);
}

template <int G>
struct DraftLds {
  static constexpr int kFloats = kWaves * G * (kD + 2);
};

__device__ __forceinline__ float row16_sum(float x) {
  // sum over the 16 lanes of a DPP row
  x += __shfl_xor(x, 1);
  x += __shfl_xor(x, 2);
  x += __shfl_xor(x, 4);
  x += __shfl_xor(x, 8);
  return x;
}

template <int G>
__device__ void draft_chunk(const DraftItem& it, int h, int split, float* part, float* lds) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rg = lane >> 4, dl = lane & 15;
  const int N = draft_set_size(it.n_sel, it.sel_len, it.L);
  const int cl = draft_chunk_len(N);
  const int p0 = split * cl;
  const int p1 = min(p0 + cl, N);
  const int lim = min(it.sel_len, it.L);
  const int32_t* selrow = it.sel + (int64_t)h * it.sel_stride;

  u32x4 qv[G];
#pragma unroll
  for (int g = 0; g < G; ++g)
    qv[g] = *reinterpret_cast<const u32x4*>(it.q + (int64_t)(h * G + g) * kD + 8 * dl);

  float m[G], l[G], o[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = kNegInf;
    l[g] = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) o[g][c] = 0.f;
  }

  const size_t page_elems = (size_t)kPage * kD;
  for (int base = p0 + 16 * wave; base < p1; base += 16 * kWaves) {
    int tok[4];
    bool ok[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int p = base + 4 * e + rg;
      ok[e] = false;
      tok[e] = 0;
      if (p < p1) {
        if (p < it.n_sel) {
          const int j = selrow[p];
          if (j < 0 || j >= it.sel_len) set_error(it.err, SSPEC_DEV_ERR_SEL_RANGE);
          ok[e] = (j >= 0 && j < lim);
          tok[e] = ok[e] ? j : 0;
        } else {
          tok[e] = it.sel_len + (p - it.n_sel);
          ok[e] = true;
        }
      }
    }
    u32x4 kr[4], vr[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (ok[e]) {
        int phys = it.bt[tok[e] / kPage];
        if (phys < 0 || phys >= it.num_pages) {
          set_error(it.err, SSPEC_DEV_ERR_PAGE_RANGE);
          phys = 0;
        }
        const size_t off = ((size_t)phys * it.hkv + h) * page_elems + (size_t)(tok[e] % kPage) * kD + 8 * dl;
        kr[e] = *reinterpret_cast<const u32x4*>(it.kp + off);
        vr[e] = *reinterpret_cast<const u32x4*>(it.vp + off);
      } else {
        kr[e] = u32x4{0, 0, 0, 0};
        vr[e] = u32x4{0, 0, 0, 0};
      }
    }
    float x[4][G];
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float d = 0.f;
        d = dot2_bf16(qv[g][0], kr[e][0], d);
        d = dot2_bf16(qv[g][1], kr[e][1], d);
        d = dot2_bf16(qv[g][2], kr[e][2], d);
        d = dot2_bf16(qv[g][3], kr[e][3], d);
        d = row16_sum(d);
        x[e][g] = ok[e] ? d * it.scale : kNegInf;
      }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float mx = fmaxf(fmaxf(x[0][g], x[1][g]), fmaxf(x[2][g], x[3][g]));
      const float mnew = fmaxf(m[g], mx);
      if (mnew == kNegInf) continue;
      const float mb = mnew * kLog2e;
      const float alpha = fast_exp2(m[g] * kLog2e - mb);
      float p[4];
      float ps = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        p[e] = fast_exp2(x[e][g] * kLog2e - mb);
        ps += p[e];
      }
      l[g] = l[g] * alpha + ps;
      m[g] = mnew;
#pragma unroll
      for (int c = 0; c < 8; c += 2) {
        float a0 = o[g][c] * alpha, a1 = o[g][c + 1] * alpha;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t w = vr[e][c >> 1];
          a0 = fmaf(p[e], bf_lo(w), a0);
          a1 = fmaf(p[e], bf_hi(w), a1);
        }
        o[g][c] = a0;
        o[g][c + 1] = a1;
      }
    }
  }

  // merge the 4 lane groups of each wave (lanes 16 and 32 apart share dims)
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float mw = fmaxf(m[g], __shfl_xor(m[g], 16));
    mw = fmaxf(mw, __shfl_xor(mw, 32));
    const float f = (mw == kNegInf) ? 0.f : fast_exp2((m[g] - mw) * kLog2e);
    float lv = l[g] * f;
    lv += __shfl_xor(lv, 16);
    lv += __shfl_xor(lv, 32);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      float v = o[g][c] * f;
      v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 32);
      o[g][c] = v;
    }
    m[g] = mw;
    l[g] = lv;
  }
  // then the 4 waves through LDS: [wave][g][m, l, o[128]]
  constexpr int RS = kD + 2;
  if (rg == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float* dst = lds + (wave * G + g) * RS;
      if (dl == 0) {
        dst[0] = m[g];
        dst[1] = l[g];
      }
#pragma unroll
      for (int c = 0; c < 8; ++c) dst[2 + 8 * dl + c] = o[g][c];
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * kD; idx += kThreads) {
    const int g = idx / kD, d = idx % kD;
    float ms = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) ms = fmaxf(ms, lds[(w * G + g) * RS]);
    float ls = 0.f, acc = 0.f;
    if (ms != kNegInf) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float* s = lds + (w * G + g) * RS;
        const float f = fast_exp2((s[0] - ms) * kLog2e);
        ls += s[1] * f;
        acc += s[2 + d] * f;
      }
    }
    if (part == nullptr) {
      const float inv = ls > 0.f ? 1.f / ls : 0.f;
      it.out[(int64_t)(h * G + g) * kD + d] = (uint16_t)f2bf_bits(acc * inv);
      if (d == 0 && it.lse) it.lse[h * G + g] = ls > 0.f ? ms + __logf(ls) : kNegInf;
    } else {
      float* dst = part + (int64_t)g * kPartStride;
      if (d == 0) {
        dst[0] = ms;
        dst[1] = ls;
      }
      dst[2 + d] = acc;
    }
  }
  __syncthreads();
}

// Merge draft partials [nsplit][G][kPartStride] of one (item, KV head).
template <int G>
__device__ void draft_combine(const DraftItem& it, int h, const float* parts, int nsplit) {
  for (int idx = threadIdx.x; idx < G * kD; idx += kThreads) {
    const int g = idx / kD, d = idx % kD;
    float ms = kNegInf;
    for (int s = 0; s < nsplit; ++s) ms = fmaxf(ms, parts[((int64_t)s * G + g) * kPartStride]);
    float ls = 0.f, acc = 0.f;
    if (ms != kNegInf) {
      for (int s = 0; s < nsplit; ++s) {
        const float* p = parts + ((int64_t)s * G + g) * kPartStride;
        const float f = fast_exp2((p[0] - ms) * kLog2e);
        ls += p[1] * f;
        acc += p[2 + d] * f;
      }
    }
    const float inv = ls > 0.f ? 1.f / ls : 0.f;
    it.out[(int64_t)(h * G + g) * kD + d] = (uint16_t)f2bf_bits(acc * inv);
    if (d == 0 && it.lse) it.lse[h * G + g] = ls > 0.f ? ms + __logf(ls) : kNegInf;
  }
}

}  // namespace sspec

// Verify attention with the logit + LSE dump [talk notes "Accelerating
// Large-Scale Reasoning Model Inference with Sparse Self-Speculative
// Decoding", section PillarAttn, paper §4.1: the verify kernel emits the
// attention scores as logits and log-sum-exp while it computes full
// attention].
//
// One task = (request, KV head, chunk of keys).  The G query heads of the
// KV head's group times the k+1 verify queries form M = G*(k+1) rows, padded
// to NQT tiles of 16.  Per pair of pages (32 keys) a wave does:
//   S^T = K * Q^T   on 16x16x32 bf16 MFMA: the key page (row-major, 256 B
//                   per token) is the A operand straight from global memory,
//                   Q^T the B operand kept in registers;
//   scale, causal mask, store the logits (fp32, 16 B per lane);
//   online softmax per query column (max across the 4 lane groups);
//   O^T += V^T * P^T  on 16x16x32 MFMA: P^T comes out of the S^T accumulator
//                   layout unchanged; V^T is built in registers from 16-byte
//                   row loads by assigning O^T row i of d-tile n to
//                   d = 8*i + n, so no LDS transpose is needed.
// The 4 waves of the work-group take page pairs round-robin and merge their
// (max, sum, O) states through LDS at the end of the chunk.
#pragma once

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

// LDS needed by verify_chunk / verify_combine (floats).
template <int NQT>
struct VerifyLds {
  static constexpr int kObufStride = kD + 4;
  static constexpr int kFloats = NQT * 16 * kObufStride + 2 * kWaves * NQT * 16 + 2 * NQT * 16;
};

__device__ __forceinline__ uint32_t sel_half(uint32_t lo_src, uint32_t hi_src, int odd) {
  // pack element (odd ? high : low) half of lo_src into bits 0..15 and the
  // same half of hi_src into bits 16..31
  return odd ? __builtin_amdgcn_perm(hi_src, lo_src, 0x07060302u)
             : __builtin_amdgcn_perm(hi_src, lo_src, 0x05040100u);
}

__device__ __forceinline__ int load_page(const int32_t* bt, int lp, int num_pages, uint32_t* err) {
  int phys = bt[lp];
  if (phys < 0 || phys >= num_pages) {
    set_error(err, SSPEC_DEV_ERR_PAGE_RANGE);
    phys = 0;
  }
  return phys;
}

// Writes the chunk's merged state: if `part` is null the final O/LSE (the
// chunk is the whole context), otherwise the partial [M][m, l, o[128]].
template <int NQT>
__device__ void verify_chunk(const VerifyItem& it, int h, int split, float* part, float* lds) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int M = it.M, kp1 = it.kp1;
  const int cl = verify_chunk_len(it.L);
  const int t0 = split * cl;
  const int t1 = min(t0 + cl, it.L);
  const int pg0 = t0 / kPage, pg1 = cdiv(t1, kPage);
  const int npairs = cdiv(pg1 - pg0, 2);

  // Q^T operand: tile qt, k-block s -> row m = 16*qt + col, d = 32*s + 8*grp .. +7
  bf16x8 qop[NQT][4];
  int lim[NQT];
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt) {
    const int m = 16 * qt + col;
    if (m < M) {
      const int gi = m / kp1, i = m - gi * kp1;
      const uint16_t* qrow = it.q + (int64_t)i * it.q_row_stride + (int64_t)(h * it.G + gi) * kD;
#pragma unroll
      for (int s = 0; s < 4; ++s)
        qop[qt][s] = as_bf16x8(*reinterpret_cast<const u32x4*>(qrow + 32 * s + 8 * grp));
      lim[qt] = it.L - kp1 + i;
    } else {
#pragma unroll
      for (int s = 0; s < 4; ++s) qop[qt][s] = as_bf16x8(u32x4{0, 0, 0, 0});
      lim[qt] = -1;
    }
  }

  float mrun[NQT], lrun[NQT];
  f32x4 o[NQT][8];
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt) {
    mrun[qt] = kNegInf;
    lrun[qt] = 0.f;
#pragma unroll
    for (int n = 0; n < 8; ++n) o[qt][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const size_t page_elems = (size_t)kPage * kD;
  for (int pp = wave; pp < npairs; pp += kWaves) {
    const int pa = pg0 + 2 * pp;
    const bool has_b = pa + 1 < pg1;
    const int phys_a = load_page(it.bt, pa, it.num_pages, it.err);
    const int phys_b = has_b ? load_page(it.bt, pa + 1, it.num_pages, it.err) : phys_a;
    const uint16_t* ka = it.kp + ((size_t)phys_a * it.hkv + h) * page_elems;
    const uint16_t* kb = it.kp + ((size_t)phys_b * it.hkv + h) * page_elems;
    const uint16_t* va = it.vp + ((size_t)phys_a * it.hkv + h) * page_elems;
    const uint16_t* vb = it.vp + ((size_t)phys_b * it.hkv + h) * page_elems;

    u32x4 kr[2][4], vr[2][4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      kr[0][s] = *reinterpret_cast<const u32x4*>(ka + col * kD + 32 * s + 8 * grp);
      kr[1][s] = *reinterpret_cast<const u32x4*>(kb + col * kD + 32 * s + 8 * grp);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      vr[0][e] = *reinterpret_cast<const u32x4*>(va + (4 * grp + e) * kD + 8 * col);
      vr[1][e] = *reinterpret_cast<const u32x4*>(vb + (4 * grp + e) * kD + 8 * col);
    }
    // keys past the context (tail of the last page) or a missing second
    // page: zero V so that 0 * garbage cannot make NaN
#pragma unroll
    for (int pg = 0; pg < 2; ++pg)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = (pa + pg) * kPage + 4 * grp + e;
        if (t >= it.L || (pg == 1 && !has_b)) vr[pg][e] = u32x4{0, 0, 0, 0};
      }

    f32x4 sacc[2][NQT];
#pragma unroll
    for (int pg = 0; pg < 2; ++pg)
#pragma unroll
      for (int qt = 0; qt < NQT; ++qt) {
        f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) a = mfma16x16x32(as_bf16x8(kr[pg][s]), qop[qt][s], a);
        sacc[pg][qt] = a;
      }

    // scale + causal mask + dump
#pragma unroll
    for (int pg = 0; pg < 2; ++pg) {
      const int tb = (pa + pg) * kPage + 4 * grp;
#pragma unroll
      for (int qt = 0; qt < NQT; ++qt) {
        f32x4 x;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float v = sacc[pg][qt][r] * it.scale;
          x[r] = (tb + r <= lim[qt]) ? v : kNegInf;
        }
        sacc[pg][qt] = x;
        const int m = 16 * qt + col;
        if (m < M && (pg == 0 || has_b)) {
          float* dst = it.dump + (int64_t)(h * M + m) * it.lstride + tb;
          *reinterpret_cast<f32x4*>(dst) = x;
        }
      }
    }

    // online softmax + PV
    uint32_t pop[NQT][4];
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) {
      float mx = kNegInf;
#pragma unroll
      for (int pg = 0; pg < 2; ++pg)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sacc[pg][qt][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mnew = fmaxf(mrun[qt], mx);
      float p[2][4];
      if (mnew == kNegInf) {
#pragma unroll
        for (int pg = 0; pg < 2; ++pg)
#pragma unroll
          for (int r = 0; r < 4; ++r) p[pg][r] = 0.f;
      } else {
        const float mb = mnew * kLog2e;
        const float alpha = fast_exp2(mrun[qt] * kLog2e - mb);  // 0 when mrun = -inf
        float ps = 0.f;
#pragma unroll
        for (int pg = 0; pg < 2; ++pg)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            p[pg][r] = fast_exp2(sacc[pg][qt][r] * kLog2e - mb);
            ps += p[pg][r];
          }
        lrun[qt] = lrun[qt] * alpha + ps;
        if (alpha != 1.f) {
#pragma unroll
          for (int n = 0; n < 8; ++n) o[qt][n] *= alpha;
        }
        mrun[qt] = mnew;
      }
      pop[qt][0] = pack_bf2(p[0][0], p[0][1]);
      pop[qt][1] = pack_bf2(p[0][2], p[0][3]);
      pop[qt][2] = pack_bf2(p[1][0], p[1][1]);
      pop[qt][3] = pack_bf2(p[1][2], p[1][3]);
    }

#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const int w = n >> 1, odd = n & 1;
      u32x4 a;
      a[0] = sel_half(vr[0][0][w], vr[0][1][w], odd);
      a[1] = sel_half(vr[0][2][w], vr[0][3][w], odd);
      a[2] = sel_half(vr[1][0][w], vr[1][1][w], odd);
      a[3] = sel_half(vr[1][2][w], vr[1][3][w], odd);
#pragma unroll
      for (int qt = 0; qt < NQT; ++qt)
        o[qt][n] = mfma16x16x32(as_bf16x8(a), as_bf16x8(u32x4{pop[qt][0], pop[qt][1], pop[qt][2], pop[qt][3]}), o[qt][n]);
    }
  }

  // ---- merge the 4 waves' states through LDS
  constexpr int OS = VerifyLds<NQT>::kObufStride;
  float* obuf = lds;                                  // [NQT*16][OS]
  float* mw = obuf + NQT * 16 * OS;                   // [kWaves][NQT*16]
  float* lw = mw + kWaves * NQT * 16;                 // [kWaves][NQT*16]
  float* mst = lw + kWaves * NQT * 16;                // [NQT*16]
  float* lst = mst + NQT * 16;                        // [NQT*16]
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt) {
    float l = lrun[qt];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if (grp == 0) {
      mw[wave * NQT * 16 + 16 * qt + col] = mrun[qt];
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
        const float f = (ms == kNegInf) ? 0.f : fast_exp2((mrun[qt] - ms) * kLog2e);
#pragma unroll
        for (int n = 0; n < 8; ++n)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int d = 8 * (4 * grp + r) + n;
            const float v = o[qt][n][r] * f;
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
      const int gi = m / kp1, i = m - gi * kp1, g = h * it.G + gi;
      uint2 pk;
      pk.x = pack_bf2(src[0] * inv, src[1] * inv);
      pk.y = pack_bf2(src[2] * inv, src[3] * inv);
      *reinterpret_cast<uint2*>(it.out + (int64_t)i * it.out_row_stride + (int64_t)g * kD + d4) = pk;
      if (d4 == 0) it.lse[(int64_t)i * it.lse_row_stride + g] = ls > 0.f ? mst[m] + __logf(ls) : kNegInf;
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

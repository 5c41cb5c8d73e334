// PillarAttn selection [talk notes "Accelerating Large-Scale Reasoning Model
// Inference with Sparse Self-Speculative Decoding", section PillarAttn,
// paper §4.1: scores are recovered from the verify kernel's logit + LSE
// dump, averaged over the draft queries and over the query heads of each
// GQA group, and the Top-K critical tokens are kept per KV head].
//
// score_chunk: S[j] = mean over the M = G*(k+1) rows of exp(logit - LSE),
//   16-byte coalesced reads of the dump, one float per key written.
// select_topk: K = min(L, ceil(s*L)) largest S per (request, KV head).
//   S >= 0, so its IEEE bit patterns order like unsigned integers: a 4-pass
//   8-bit radix select finds the K-th largest key exactly, then one
//   block-scan pass emits the winners in ascending index order (keys equal
//   to the threshold are taken lowest index first).
#pragma once

#include "sspec_common.hpp"

namespace sspec {

struct ScoreItem {
  const float* dump;     // row (g, i) at dump + (g*kp1 + i)*lstride
  int64_t lstride;
  const float* lse;      // query row i, head g at lse + i*lse_row_stride + g
  int64_t lse_row_stride;
  int hq, kp1, G, M, L;
  float* scores;         // S row of (item, h): scores + h*sstride
  int64_t sstride;
};

constexpr int kSelectLdsFloats = kWaves * 256 + 3 * kWaves + 16 + kMaxRows;

// Exclusive block scan of one int per thread; *total gets the block sum.
__device__ inline int block_excl_scan(int v, int* tmp /*[kWaves]*/, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) tmp[wave] = x;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const int t = tmp[w];
    base += (w < wave) ? t : 0;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return base + x - v;
}

__device__ void score_chunk(const ScoreItem& it, int h, int c, float* lds) {
  float* lse2 = lds;  // [M] LSE in log2 units
  const int M = it.M;
  for (int m = threadIdx.x; m < M; m += kThreads) {
    const int gi = m / it.kp1, i = m - gi * it.kp1;
    lse2[m] = it.lse[(int64_t)i * it.lse_row_stride + h * it.G + gi] * kLog2e;
  }
  __syncthreads();
  const int t0 = c * kScoreChunk;
  const int t1 = min(t0 + kScoreChunk, it.L);
  const float invM = 1.f / (float)M;
  const float* base = it.dump + (int64_t)h * M * it.lstride;
  float* srow = it.scores + (int64_t)h * it.sstride;
  for (int j = t0 + 4 * threadIdx.x; j < t1; j += 4 * kThreads) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int m = 0; m < M; ++m) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(base + (int64_t)m * it.lstride + j);
      const float l2 = lse2[m];
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] += fast_exp2(fmaf(x[e], kLog2e, -l2));
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (j + e >= t1) acc[e] = 0.f;   // keys past the context score 0
    *reinterpret_cast<f32x4*>(srow + j) = acc * invM;
  }
  __syncthreads();
}

// Top-K of one (item, KV head) from its score row.  Writes sel[0..K).
__device__ void select_topk(const float* srow, int L, int K, int32_t* sel, float* ldsf) {
  int* hist = reinterpret_cast<int*>(ldsf);          // [kWaves][256]
  int* tmp = hist + kWaves * 256;                    // [kWaves] scan scratch
  int* shared = tmp + 3 * kWaves;                    // [16] broadcast slots
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t* key = reinterpret_cast<const uint32_t*>(srow);

  uint32_t prefix = 0, mask = 0;
  int remaining = K;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int b = threadIdx.x; b < kWaves * 256; b += kThreads) hist[b] = 0;
    __syncthreads();
    for (int j = threadIdx.x; j < L; j += kThreads) {
      const uint32_t u = key[j];
      if ((u & mask) == prefix) atomicAdd(&hist[wave * 256 + ((u >> shift) & 255u)], 1);
    }
    __syncthreads();
    // thread t owns bin 255 - t: an inclusive scan over t is a suffix count
    const int bin = 255 - threadIdx.x;
    int cnt = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) cnt += hist[w * 256 + bin];
    int total;
    const int above = block_excl_scan(cnt, tmp, &total);   // keys in bins > bin
    if (above < remaining && above + cnt >= remaining) {
      shared[0] = bin;
      shared[1] = above;
    }
    __syncthreads();
    const uint32_t b = (uint32_t)shared[0];
    remaining -= shared[1];
    prefix |= b << shift;
    mask |= 255u << shift;
    __syncthreads();
  }
  const uint32_t T = prefix;       // key of the K-th largest score
  const int need_eq = remaining;   // how many keys equal to T are taken

  // ascending emit, 4 keys per thread per tile of 1024
  int out_base = 0, eq_base = 0;
  for (int j0 = 0; j0 < L; j0 += 4 * kThreads) {
    const int j = j0 + 4 * threadIdx.x;
    uint32_t u[4];
    int gt = 0, eq = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      u[e] = (j + e < L) ? key[j + e] : 0u;
      const bool in = j + e < L;
      gt += (in && u[e] > T);
      eq += (in && u[e] == T);
    }
    (void)gt;
    int eq_tot;
    const int eq_before = eq_base + block_excl_scan(eq, tmp, &eq_tot);
    bool take[4];
    int cnt = 0, er = eq_before;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool in = j + e < L;
      bool t = in && u[e] > T;
      if (in && u[e] == T) {
        t = er < need_eq;
        ++er;
      }
      take[e] = t;
      cnt += t;
    }
    int tot;
    int pos = out_base + block_excl_scan(cnt, tmp, &tot);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (take[e]) {
        if (pos < K) sel[pos] = j + e;  // never past the K slots of this row
        ++pos;
      }
    out_base += tot;
    eq_base += eq_tot;
  }
  (void)lane;
}

}  // namespace sspec

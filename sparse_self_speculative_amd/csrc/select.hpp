// PillarAttn selection [talk notes "Accelerating Large-Scale Reasoning Model
// Inference with Sparse Self-Speculative Decoding", section PillarAttn,
// paper §4.1: scores are recovered from the verify kernel's logit + LSE
// dump, averaged over the draft queries and over the query heads of each
// GQA group, and the Top-K critical tokens are kept per KV head].
//
// score_wave_chunk (one wave, kScoreChunk keys of one (item, KV head)):
//   S[j] = mean over the M = G*(k+1) rows of exp(logit - LSE), read from the
//   dump with 16-byte device-coherent loads; S is stored, and the 11-bit
//   histogram of the S bit patterns' top digit (bits 30..20) is added into
//   the (item, KV head)'s global histogram.
// select_wave (one wave, run by whichever wave scores an (item, KV head)'s
//   last chunk): K = min(L, ceil(s*L)) largest S.  S >= 0, so IEEE bit
//   patterns order like unsigned integers.  The global histogram gives the
//   bin B1 that holds the K-th largest key; one pass collects the keys of
//   bin B1 into LDS (when they fit), two radix passes over those candidates
//   (bits 19..9, 8..0) give the exact K-th largest key T; a final pass emits
//   every key > T and the first keys == T (lowest index first), in ascending
//   index order.  When bin B1 holds more keys than fit in LDS, the two radix
//   passes read all keys instead.
#pragma once

#include "ring.hpp"
#include "sspec_common.hpp"

namespace sspec {

constexpr int kCandCap = 4096;     // candidate keys held in LDS
// Per-wave LDS of a score / select task: histogram, then candidates.
struct SelectWaveLds {
  static constexpr int kHistOff = 0;
  static constexpr int kCandOff = kHistBins * 4;
  static constexpr int kBytes = kCandOff + kCandCap * 4;
};
static_assert(SelectWaveLds::kBytes <= kRing * kSlotBytes, "select LDS must fit in the ring area");

struct ScoreItem {
  const float* dump;     // row (g, i) at dump + (g*kp1 + i)*lstride
  int64_t lstride;
  const float* lse;      // query row i, head g at lse + i*lse_row_stride + g
  int64_t lse_row_stride;
  int kp1, G, M, L;
  float* scores;         // S row of (item, h): scores + h*sstride (sstride multiple of kScoreChunk)
  int64_t sstride;
  uint32_t* hist;        // top-digit histogram of (item, h): hist + h*kHistBins
};

__device__ SSPEC_TASK void score_wave_chunk(const ScoreItem& it, int h, int c, char* wlds) {
  const int lane = (int)lane_id();
  const int M = it.M;
  const int t0 = c * kScoreChunk;
  const int t1 = min(t0 + kScoreChunk, it.L);
  // LSE of rows lane and lane + 64, in log2 units
  float l2[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int m = lane + 64 * e;
    l2[e] = 0.f;
    if (m < M) {
      const int gi = m / it.kp1, i = m - gi * it.kp1;
      l2[e] = ld_coh(it.lse + (int64_t)i * it.lse_row_stride + h * it.G + gi) * kLog2e;
    }
  }
  const float* base = wave_uniform(it.dump + (int64_t)h * M * it.lstride + t0);
  // the range ends at the last row's t1: nothing past the dump is read
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(base, (uint32_t)(((int64_t)(M - 1) * it.lstride + (t1 - t0)) * 4));
  f32x4 acc[4];
#pragma unroll
  for (int cc = 0; cc < 4; ++cc) acc[cc] = f32x4{0.f, 0.f, 0.f, 0.f};
  const uint32_t lrow = (uint32_t)it.lstride * 4u;
#pragma unroll 4
  for (int m = 0; m < M; ++m) {
    const float lmf = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m < 64 ? l2[0] : l2[1]), m & 63));
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      const f32x4 x = ld_coh4(rs, (uint32_t)m * lrow + (uint32_t)(256 * cc + 4 * lane) * 4u);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[cc][e] += fast_exp2(fmaf(x[e], kLog2e, -lmf));
    }
  }
  const float invM = 1.f / (float)M;
  float* srow = it.scores + (int64_t)h * it.sstride + t0;
  int* hist = reinterpret_cast<int*>(wlds + SelectWaveLds::kHistOff);
#pragma unroll
  for (int b = 0; b < kHistBins / kWave; b += 4)
    *reinterpret_cast<u32x4*>(hist + kHistBins / kWave * lane + b) = u32x4{0, 0, 0, 0};
#pragma unroll
  for (int cc = 0; cc < 4; ++cc) {
    const int j = 256 * cc + 4 * lane;   // relative to t0
    f32x4 sv;
#pragma unroll
    for (int e = 0; e < 4; ++e) sv[e] = (t0 + j + e < t1) ? acc[cc][e] * invM : 0.f;   // past the context: 0
    st_coh4(srow + j, sv);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (t0 + j + e < t1) atomicAdd(&hist[__float_as_uint(sv[e]) >> 20], 1);
  }
  // flush the nonzero bins (lane owns 32 consecutive bins)
  uint32_t* gh = it.hist + (int64_t)h * kHistBins;
#pragma unroll
  for (int b = 0; b < kHistBins / kWave; b += 4) {
    const int bin = kHistBins / kWave * lane + b;
    const u32x4 v = *reinterpret_cast<const u32x4*>(hist + bin);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (v[e]) __hip_atomic_fetch_add(gh + bin + e, v[e], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Bin (of nbins, highest first) that holds the need-th largest key counted in
// the LDS histogram, and the number of keys in higher bins.
__device__ __forceinline__ void hist_find(const int* hist, int nbins, int need, int& bin, int& above) {
  const int lane = (int)lane_id();
  const int per = nbins / kWave;
  const int top = nbins - per * lane;   // this lane owns bins [top - per, top)
  int s = 0;
  for (int b = 0; b < per; ++b) s += hist[top - 1 - b];
  int total;
  const int pre = wave_excl_scan(s, &total);
  const bool mine = pre < need && pre + s >= need;
  int fb = 0, fa = 0;
  if (mine) {
    int acc = pre;
    for (int b = 0; b < per; ++b) {
      const int cnt = hist[top - 1 - b];
      if (acc + cnt >= need) {
        fb = top - 1 - b;
        fa = acc;
        break;
      }
      acc += cnt;
    }
  }
  const uint64_t who = __ballot(mine);
  if (who == 0) {   // inconsistent counts (cannot happen for a valid need)
    bin = 0;
    above = 0;
    return;
  }
  const int src = __builtin_ctzll(who);
  bin = __builtin_amdgcn_readlane(fb, src);
  above = __builtin_amdgcn_readlane(fa, src);
}

__device__ __forceinline__ void hist_clear(int* hist) {
  const int lane = (int)lane_id();
#pragma unroll
  for (int b = 0; b < kHistBins / kWave; b += 4)
    *reinterpret_cast<u32x4*>(hist + kHistBins / kWave * lane + b) = u32x4{0, 0, 0, 0};
}

// Histogram, into LDS, of digit (u >> shift) & dmask of the keys u of
// [0, L) with (u & fmask) == fval.
__device__ void hist_pass_global(__amdgpu_buffer_rsrc_t rs, int L, uint32_t fmask, uint32_t fval, int shift,
                                 uint32_t dmask, int* hist) {
  const int lane = (int)lane_id();
  hist_clear(hist);
  for (int j0 = 0; j0 < L; j0 += 4 * kWave * 4) {
    u32x4 u[4];
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) u[cc] = ld_coh4u(rs, (uint32_t)(j0 + 256 * cc + 4 * lane) * 4u);
#pragma unroll
    for (int cc = 0; cc < 4; ++cc)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = j0 + 256 * cc + 4 * lane + e;
        if (j < L && (u[cc][e] & fmask) == fval) atomicAdd(&hist[(u[cc][e] >> shift) & dmask], 1);
      }
  }
}

// Top-K of one score row (written in this launch by other waves: coherent
// loads).  ghist: the row's top-digit histogram, cleared here after use.
__device__ SSPEC_TASK void select_wave(const float* srow, int L, int K, uint32_t* ghist, int32_t* sel, char* wlds) {
  const int lane = (int)lane_id();
  int* hist = reinterpret_cast<int*>(wlds + SelectWaveLds::kHistOff);
  uint32_t* cand = reinterpret_cast<uint32_t*>(wlds + SelectWaveLds::kCandOff);
  srow = wave_uniform(srow);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(srow, (uint32_t)L * 4u);

  // ---- digit 1 (bits 30..20): from the global histogram, which is reset
#pragma unroll
  for (int b = 0; b < kHistBins / kWave; b += 4) {
    const int bin = kHistBins / kWave * lane + b;
    u32x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = ld_coh_u(ghist + bin + e);
    *reinterpret_cast<u32x4*>(hist + bin) = v;
#pragma unroll
    for (int e = 0; e < 4; ++e) st_coh_u(ghist + bin + e, 0u);
  }
  if (K <= 0) return;
  int b1, above;
  hist_find(hist, kHistBins, K, b1, above);
  int need = K - above;
  const int n1 = hist[b1];
  int b2, b3;
  if (n1 <= kCandCap) {
    // ---- collect the keys of bin b1
    int nc = 0;
    for (int j0 = 0; j0 < L; j0 += 4 * kWave * 4) {
      u32x4 u[4];
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) u[cc] = ld_coh4u(rs, (uint32_t)(j0 + 256 * cc + 4 * lane) * 4u);
#pragma unroll
      for (int cc = 0; cc < 4; ++cc)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = j0 + 256 * cc + 4 * lane + e;
          const bool in = j < L && (u[cc][e] >> 20) == (uint32_t)b1;
          const uint64_t bal = __ballot(in);
          const int pos = nc + (int)lanemask_lt_count(bal);
          if (in && pos < kCandCap) cand[pos] = u[cc][e];
          nc += __builtin_popcountll(bal);
        }
    }
    nc = min(nc, kCandCap);
    // ---- digit 2 (bits 19..9) over the candidates
    hist_clear(hist);
    for (int i = lane; i < nc; i += kWave) atomicAdd(&hist[(cand[i] >> 9) & 2047u], 1);
    hist_find(hist, kHistBins, need, b2, above);
    need -= above;
    // ---- digit 3 (bits 8..0)
    hist_clear(hist);
    for (int i = lane; i < nc; i += kWave) {
      const uint32_t u = cand[i];
      if (((u >> 9) & 2047u) == (uint32_t)b2) atomicAdd(&hist[u & 511u], 1);
    }
    hist_find(hist, 512, need, b3, above);
    need -= above;
  } else {
    hist_pass_global(rs, L, 0xfff00000u, (uint32_t)b1 << 20, 9, 2047u, hist);
    hist_find(hist, kHistBins, need, b2, above);
    need -= above;
    hist_pass_global(rs, L, 0xfffffe00u, ((uint32_t)b1 << 20) | ((uint32_t)b2 << 9), 0, 511u, hist);
    hist_find(hist, 512, need, b3, above);
    need -= above;
  }
  const uint32_t T = ((uint32_t)b1 << 20) | ((uint32_t)b2 << 9) | (uint32_t)b3;
  const int need_eq = need;   // keys equal to T to take, lowest index first

  // ---- emit in ascending index order
  int out = 0, eq_seen = 0;
  for (int j0 = 0; j0 < L && out < K; j0 += 4 * kWave * 4) {
    u32x4 u[4];
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) u[cc] = ld_coh4u(rs, (uint32_t)(j0 + 256 * cc + 4 * lane) * 4u);
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      const int jb = j0 + 256 * cc + 4 * lane;
      bool gt[4], eq[4];
      uint64_t beq[4];
      int eq_tot = 0;
      uint32_t eq_lt = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool in = jb + e < L;
        gt[e] = in && u[cc][e] > T;
        eq[e] = in && u[cc][e] == T;
        beq[e] = __ballot(eq[e]);
        eq_tot += __builtin_popcountll(beq[e]);
        eq_lt += lanemask_lt_count(beq[e]);
      }
      bool take[4];
      int rank = eq_seen + (int)eq_lt;
      uint64_t btk[4];
      int tk_tot = 0;
      uint32_t tk_lt = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        take[e] = gt[e];
        if (eq[e]) {
          take[e] = rank < need_eq;
          ++rank;
        }
        btk[e] = __ballot(take[e]);
        tk_tot += __builtin_popcountll(btk[e]);
        tk_lt += lanemask_lt_count(btk[e]);
      }
      int pos = out + (int)tk_lt;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (take[e]) {
          if (pos < K) sel[pos] = jb + e;   // never past the K slots of this row
          ++pos;
        }
      out += tk_tot;
      eq_seen += eq_tot;
    }
  }
}

}  // namespace sspec

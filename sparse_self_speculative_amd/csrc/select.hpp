// PillarAttn selection [talk notes "Accelerating Large-Scale Reasoning Model
// Inference with Sparse Self-Speculative Decoding", section PillarAttn,
// paper §4.1: scores are recovered from the verify kernel's logit + LSE
// dump, averaged over the draft queries and over the query heads of each
// GQA group, and the Top-K critical tokens are kept per KV head].
//
// score_wave_chunk (one wave, one chunk of keys of one (item, KV head)):
//   S[j] = mean over the M = G*(k+1) rows of exp(logit - LSE), read from the
//   page-blocked dump with 16-byte device-coherent loads; S is stored, and
//   the 11-bit
//   histogram of the S bit patterns' top digit (bits 30..20) is added into
//   the (item, KV head)'s global histogram.
// Selection, K = min(L, ceil(s*L)) largest S of a row: S >= 0, so IEEE
//   bit patterns order like unsigned integers.  The row's global histogram
//   (complete once every chunk has added to it) gives the bin b1 that holds
//   the K-th largest key (select_prepare).  Every key is classified against
//   b1 into two bitmaps, keys above b1 (all selected) and keys in b1 (the
//   candidates), from a copy of the scores' top 16 bits that the score
//   chunks also write (collect_bits).  select_final gathers the candidates,
//   resolves the exact K-th key T by two radix digits (bits 19..9, 8..0),
//   and writes every key > T and the first keys == T (lowest index first) in
//   ascending index order.  When bin b1 holds more keys than kFastCap,
//   select_wave runs instead: it collects the bin's keys into LDS (or, past
//   kCandCap keys, makes two radix passes over all keys) and emits in one
//   more pass.
#pragma once

#include "ring.hpp"
#include "sspec_common.hpp"

namespace sspec {

constexpr int kCandCap = 4096;     // candidate keys held in LDS (select_wave)
constexpr int kFastCap = 2048;     // candidates held in LDS (bitmap selection)
constexpr int kGroups = 16;        // 16-byte loads per lane in flight in a select_wave pass

// Per-wave LDS of a score / select task: histogram, then the candidates --
// keys (select_wave), or keys and indices (select_final).
struct SelectWaveLds {
  static constexpr int kHistOff = 0;
  static constexpr int kCandOff = kHistBins * 4;
  static constexpr int kCkOff = kHistBins * 4;
  static constexpr int kCiOff = kCkOff + kFastCap * 4;
  static constexpr int kBytes = kCiOff + kFastCap * 4;
  static_assert(kCandOff + kCandCap * 4 <= kBytes, "select_wave's candidates fit");
};

struct ScoreItem {
  const float* dump;     // page-blocked logits of the item: (h, key j, row m) at
                         // dump + (h*lstride + 16*(j/16))*mp + 16*m + j%16
  int64_t lstride;       // keys per KV head in the dump (multiple of 16)
  int mp;                // rows per page block (round_up(M, 4))
  const float* lse;      // query row i, head g at lse + i*lse_row_stride + g
  int64_t lse_row_stride;
  int kp1, G, M, L;
  float* scores;         // S row of (item, h): scores + h*sstride (sstride multiple of kScoreChunk)
  uint16_t* tops;        // top 16 bits of each S, row of (item, h): tops + h*sstride
  int64_t sstride;
  int chunk;             // keys per score task (divides kScoreChunk)
  uint32_t* hist;        // top-digit histogram of (item, h): hist + h*kHistBins
};

// Scores of one chunk, NI = cdiv(mp, 16) 1 KB loads per page block.  In load
// i of a page, lane l holds rows 16*i + l/4, keys 4*(l%4) .. +3 of the page
// (the block is [rows][16 keys]), so exp(logit - LSE) is summed over i in
// the lane and then over the 16 lanes that hold the same keys (DPP row
// rotations by 4 and 8, then v_permlane16/32_swap).  Lane l keeps the sums of
// page p when l/4 == p%16; every 16 pages its 4 scores go out as one
// lane-contiguous store.  Pages are fetched in batches of 24/NI, two batches
// in flight.  Rows >= M (and past the block) get LSE = +inf, i.e. weight 0.
template <int NI>
__device__ __forceinline__ void score_chunk_ni(const ScoreItem& it, int h, int c, char* wlds) {
  constexpr int PB = 24 / NI;   // pages per batch
  const int lane = (int)lane_id();
  const int M = it.M, mp = it.mp;
  const int t0 = c * it.chunk;
  const int t1 = min(t0 + it.chunk, it.L);
  const int npg = cdiv(t1 - t0, kPage);
  // LSE (log2 units) of rows lane and lane + 64, then of this lane's row in
  // each load
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
  float lr[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int r = 16 * i + (lane >> 2);
    const float v = __shfl(i < 4 ? l2[0] : l2[1], r & 63);
    lr[i] = r < M ? v : __builtin_huge_valf();
  }
  const float* base = wave_uniform(it.dump + ((int64_t)h * it.lstride + t0) * mp);
  const uint32_t pbytes = (uint32_t)(kPage * mp * 4);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(base, (uint32_t)npg * pbytes);
  const float invM = 1.f / (float)M;
  float* srow = it.scores + (int64_t)h * it.sstride + t0;
  const __amdgpu_buffer_rsrc_t rtop = make_rsrc(wave_uniform(it.tops + (int64_t)h * it.sstride + t0), (uint32_t)it.chunk * 2u);
  int* hist = reinterpret_cast<int*>(wlds + SelectWaveLds::kHistOff);
#pragma unroll
  for (int b = 0; b < kHistBins / kWave; b += 4)
    *reinterpret_cast<u32x4*>(hist + kHistBins / kWave * lane + b) = u32x4{0, 0, 0, 0};

  const int nb = cdiv(npg, PB);
  auto fetch = [&](f32x4 (&v)[PB][NI], int b) __attribute__((always_inline)) {
#pragma unroll
    for (int pp = 0; pp < PB; ++pp)
#pragma unroll
      for (int i = 0; i < NI; ++i)
        v[pp][i] = ld_coh4(rs, (uint32_t)(b * PB + pp) * pbytes + (uint32_t)(256 * i + 4 * lane) * 4u);
  };
  f32x4 res = {0.f, 0.f, 0.f, 0.f};   // sums of page p with p%16 == lane/4
  auto flush = [&](int p0) __attribute__((always_inline)) {   // pages p0 .. p0+15
    const int j = 16 * p0 + 4 * lane;   // relative to t0
    f32x4 sv;
#pragma unroll
    for (int q = 0; q < 4; ++q) sv[q] = (t0 + j + q < t1) ? res[q] * invM : 0.f;   // past the context: 0
    st_coh4(srow + j, sv);
    // the top halves, for the classification pass (8 bytes per lane)
    const uint32_t top01 = (__float_as_uint(sv[0]) >> 16) | (__float_as_uint(sv[1]) & 0xffff0000u);
    const uint32_t top23 = (__float_as_uint(sv[2]) >> 16) | (__float_as_uint(sv[3]) & 0xffff0000u);
    st_coh2u_buf(rtop, (uint32_t)j * 2u, top01, top23);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (t0 + j + q < t1) atomicAdd(&hist[__float_as_uint(sv[q]) >> 20], 1);
    res = f32x4{0.f, 0.f, 0.f, 0.f};
  };
  auto process = [&](f32x4 (&v)[PB][NI], int b) __attribute__((always_inline)) {
    f32x4 cur[PB][NI];
#pragma unroll
    for (int pp = 0; pp < PB; ++pp)
#pragma unroll
      for (int i = 0; i < NI; ++i) cur[pp][i] = v[pp][i];
    if (b + 2 < nb) fetch(v, b + 2);   // the next-but-one batch
#pragma unroll
    for (int pp = 0; pp < PB; ++pp) {
      const int p = b * PB + pp;
      if (p < npg) {
        f32x4 sq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q) sq[q] += fast_exp2(fmaf(cur[pp][i][q], kLog2e, -lr[i]));
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float x = sq[q];
          x += SSPEC_DPP(x, 0x124);   // row_ror:4
          x += SSPEC_DPP(x, 0x128);   // row_ror:8
          sq[q] = sum_xor32(sum_xor16(x));
        }
        if ((lane >> 2) == (p & 15)) res = sq;
        if ((p & 15) == 15 || p + 1 == npg) flush(p & ~15);
      }
    }
  };
  f32x4 va[PB][NI], vb[PB][NI];
  fetch(va, 0);
  if (nb > 1) fetch(vb, 1);
  for (int b = 0; b < nb; b += 2) {
    process(va, b);
    if (b + 1 < nb) process(vb, b + 1);
  }
  // score-row entries past the last page group are zero
  for (int j = round_up(npg, 16) * kPage + 4 * lane; j < it.chunk; j += 4 * kWave)
    st_coh4(srow + j, f32x4{0.f, 0.f, 0.f, 0.f});
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

__device__ SSPEC_TASK void score_wave_chunk(const ScoreItem& it, int h, int c, char* wlds) {
  switch (cdiv(it.mp, 16)) {
    case 1: score_chunk_ni<1>(it, h, c, wlds); break;
    case 2: score_chunk_ni<2>(it, h, c, wlds); break;
    case 3: score_chunk_ni<3>(it, h, c, wlds); break;
    case 4: score_chunk_ni<4>(it, h, c, wlds); break;
    case 5: score_chunk_ni<5>(it, h, c, wlds); break;
    case 6: score_chunk_ni<6>(it, h, c, wlds); break;
    case 7: score_chunk_ni<7>(it, h, c, wlds); break;
    default: score_chunk_ni<8>(it, h, c, wlds); break;
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
__device__ __forceinline__ void hist_pass_global(__amdgpu_buffer_rsrc_t rs, int L, uint32_t fmask, uint32_t fval, int shift,
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

// Exact threshold key T among the candidate keys ck[0, nc) (all in top-digit
// bin b1): radix digits 2 (bits 19..9) and 3 (bits 8..0); *need enters as
// the number of candidates to take and leaves as the number of keys == T to
// take.
__device__ __forceinline__ uint32_t resolve_threshold(const uint32_t* ck, int nc, int b1, int* need, int* hist) {
  const int lane = (int)lane_id();
  int b2, b3, above;
  hist_clear(hist);
  for (int i = lane; i < nc; i += kWave) atomicAdd(&hist[(ck[i] >> 9) & 2047u], 1);
  hist_find(hist, kHistBins, *need, b2, above);
  *need -= above;
  hist_clear(hist);
  for (int i = lane; i < nc; i += kWave) {
    const uint32_t u = ck[i];
    if (((u >> 9) & 2047u) == (uint32_t)b2) atomicAdd(&hist[u & 511u], 1);
  }
  hist_find(hist, 512, *need, b3, above);
  *need -= above;
  return ((uint32_t)b1 << 20) | ((uint32_t)b2 << 9) | (uint32_t)b3;
}

// ------------------------------------------------- bitmap selection ---
// Once the last score chunk of a (request, KV head) pair has completed the
// pair's top-digit histogram, the bin b1 that holds the K-th largest key is
// known (select_prepare).  Every key is classified against b1 into two
// bitmaps (keys in bins above b1, all selected; keys in bin b1, the
// candidates): per key a compare and an OR.  Then one wave resolves the
// exact K-th key among the at most kFastCap candidates and writes the
// selection in ascending index order straight from the bitmaps
// (select_final).  When bin b1 holds more keys than kFastCap, select_wave
// runs instead.
struct SelInfo {
  uint32_t b1;        // top-digit bin of the K-th largest key
  int32_t need;       // keys to take from bin b1
  int32_t n1;         // keys in bin b1
  int32_t fallback;   // 1: bin b1 too large (or K <= 0): select_wave runs instead
};
constexpr int kBitWords = kScoreChunk / 32;   // words of one kind of bitmap per kScoreChunk keys

// From the pair's top-digit histogram (complete: every chunk has added to
// it): b1, the keys needed from it, and whether the bitmap path applies.
// The histogram is cleared unless the pair falls back (select_wave then
// reads and clears it).
__device__ __forceinline__ SelInfo select_prepare(uint32_t* ghist, int K, char* wlds) {
  const int lane = (int)lane_id();
  int* hist = reinterpret_cast<int*>(wlds + SelectWaveLds::kHistOff);
  ghist = wave_uniform(ghist);
  const __amdgpu_buffer_rsrc_t rh = make_rsrc(ghist, kHistBins * 4u);
  u32x4 v[kHistBins / kWave / 4];
#pragma unroll
  for (int b = 0; b < kHistBins / kWave / 4; ++b) v[b] = ld_coh4u(rh, (uint32_t)(kHistBins / kWave * lane + 4 * b) * 4u);
#pragma unroll
  for (int b = 0; b < kHistBins / kWave / 4; ++b)
    *reinterpret_cast<u32x4*>(hist + kHistBins / kWave * lane + 4 * b) = v[b];
  SelInfo info;
  info.b1 = 0;
  info.need = 0;
  info.n1 = 0;
  info.fallback = 1;
  if (K > 0) {
    int b1, above;
    hist_find(hist, kHistBins, K, b1, above);
    info.b1 = (uint32_t)b1;
    info.need = K - above;
    info.n1 = hist[b1];
    info.fallback = info.n1 > kFastCap;
  }
  if (!info.fallback) {
#pragma unroll
    for (int b = 0; b < kHistBins / kWave / 4; ++b)
      st_coh4(reinterpret_cast<float*>(ghist + kHistBins / kWave * lane + 4 * b), f32x4{0.f, 0.f, 0.f, 0.f});
  }
  return info;
}

// OR over the 8 lanes of each aligned group of 8 (quad swaps, then the
// mirror of the half row pairs the two quads).
__device__ __forceinline__ uint32_t or_lanes8(uint32_t x) {
  x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
  x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
  x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x141, 0xF, 0xF, false);  // row_half_mirror
  return x;
}

constexpr int kTopLoads = kScoreChunk / (8 * kWave);   // 16-byte loads per lane per chunk of top halves

// Keys of one score chunk (nk of them) against b1 from their scores' top 16
// bits (S >= 0: bits 14..4 of the top half are the 11-bit bin, bits 30..20
// of S), lane l holding keys 512cc + 8l .. +7 in u[cc], into the chunk's
// bitmaps cb: bit j%32 of word j/32 in its first kBitWords words for keys in
// bins above b1 and in the next kBitWords for keys in bin b1 (the 4-lane ORs
// assemble each word).
__device__ __forceinline__ void classify_tops(const u32x4 (&u)[kTopLoads], int nk, uint32_t b1, uint32_t* cb) {
  const int lane = (int)lane_id();
#pragma unroll
  for (int cc = 0; cc < kTopLoads; ++cc) {
    // lane l holds keys 512cc + 8l .. +7: word 16cc + l/4, bits 8(l%4) .. +7
    uint32_t dn = 0, cn = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int j = 512 * cc + 8 * lane + e;
      const uint32_t bin = ((u[cc][e >> 1] >> (16 * (e & 1))) & 0xffffu) >> 4;
      const uint32_t bit = 1u << (8 * (lane & 3) + e);
      dn |= (j < nk && bin > b1) ? bit : 0u;
      cn |= (j < nk && bin == b1) ? bit : 0u;
    }
    dn |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)dn, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
    dn |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)dn, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
    cn |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)cn, 0xB1, 0xF, 0xF, false);
    cn |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)cn, 0x4E, 0xF, 0xF, false);
    if ((lane & 3) == 0) {
      st_coh_u(cb + 16 * cc + (lane >> 2), dn);
      st_coh_u(cb + kBitWords + 16 * cc + (lane >> 2), cn);
    }
  }
}

// Every chunk of a pair's row against b1, by one wave, from the top halves
// of its scores (2 bytes per key), the next seven chunks in flight while the
// current one is classified: the pass waits on memory, so halving its bytes
// and doubling the keys in flight shortens it.
__device__ SSPEC_TASK void collect_bits(const uint16_t* trow, int L, uint32_t b1, uint32_t* bits) {
  const int lane = (int)lane_id();
  // whole 16-byte loads stay inside the range (the score chunks wrote the
  // top halves of their last 256-key group whole, zero past the context)
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(wave_uniform(trow), (uint32_t)round_up(L, 8) * 2u);
  bits = wave_uniform(bits);
  const int nchunks = score_splits(L);
  auto fetch = [&](u32x4 (&u)[kTopLoads], int c) __attribute__((always_inline)) {
#pragma unroll
    for (int cc = 0; cc < kTopLoads; ++cc)
      u[cc] = ld_coh4u(rs, (uint32_t)(c * kScoreChunk + 512 * cc + 8 * lane) * 2u);
  };
  constexpr int kAhead = 7;
  u32x4 ub[kAhead + 1][kTopLoads];
#pragma unroll
  for (int j = 0; j < kAhead; ++j)
    if (j < nchunks) fetch(ub[j], j);
  for (int c = 0; c < nchunks; c += kAhead + 1) {
#pragma unroll
    for (int j = 0; j <= kAhead; ++j) {
      const int cc = c + j;
      if (cc < nchunks) {
        // the buffer of chunk cc - 1, classified just before, takes chunk cc + kAhead
        if (cc + kAhead < nchunks) fetch(ub[(j + kAhead) % (kAhead + 1)], cc + kAhead);
        classify_tops(ub[j], min(kScoreChunk, L - cc * kScoreChunk), b1, bits + (int64_t)cc * 2 * kBitWords);
      }
    }
  }
  drain_vm();   // the bitmaps are read back (coherently) by select_final
}

// After collect_bits: candidates (keys of bin b1, in index
// order) gathered from the bitmaps into LDS with their keys, the exact
// threshold T resolved among them, then the selection written in ascending
// order: every key of the "above" bitmap and the chosen candidates (keys > T
// and the first `need` keys == T, lowest index first).  bits: the pair's
// [chunks][2][kBitWords].
__device__ SSPEC_TASK void select_final(const float* srow, int L, int K, const SelInfo& info, const uint32_t* bits,
                                        int32_t* sel, char* wlds) {
  const int lane = (int)lane_id();
  int* hist = reinterpret_cast<int*>(wlds + SelectWaveLds::kHistOff);
  uint32_t* ck = reinterpret_cast<uint32_t*>(wlds + SelectWaveLds::kCkOff);
  int* ci = reinterpret_cast<int*>(wlds + SelectWaveLds::kCiOff);
  srow = wave_uniform(srow);
  bits = wave_uniform(bits);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(srow, (uint32_t)L * 4u);
  const int nchunks = score_splits(L);
  const int nwords = nchunks * kBitWords;
  // word w of kind k (0 above, 1 candidate) of the pair
  auto word_off = [&](int w, int k) __attribute__((always_inline)) -> int {
    return (w / kBitWords) * 2 * kBitWords + k * kBitWords + (w % kBitWords);
  };
  constexpr int kW = 8;   // words per lane per round
  // ---- candidates, in index order, with their keys
  int npos = 0;
  for (int w0 = 0; w0 < nwords; w0 += kW * kWave) {
    uint32_t cw[kW];
#pragma unroll
    for (int q = 0; q < kW; ++q) {
      const int w = w0 + kW * lane + q;
      cw[q] = w < nwords ? ld_coh_u(bits + word_off(w, 1)) : 0u;
    }
    int cnt = 0;
#pragma unroll
    for (int q = 0; q < kW; ++q) cnt += __builtin_popcount(cw[q]);
    int tot;
    int pos = npos + wave_excl_scan(cnt, &tot);
#pragma unroll
    for (int q = 0; q < kW; ++q) {
      uint32_t m = cw[q];
      const int w = w0 + kW * lane + q;
      while (m) {
        const int b = __builtin_ctz(m);
        m &= m - 1;
        if (pos < kFastCap) ci[pos] = 32 * w + b;
        ++pos;
      }
    }
    npos += tot;
  }
  const int nc = min(npos, kFastCap);
  // their keys: sixteen loads per lane in flight at a time
  for (int i0 = 0; i0 < nc; i0 += 16 * kWave) {
    float kv[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int i = i0 + kWave * t + lane;
      kv[t] = i < nc ? ld_coh1(rs, (uint32_t)ci[i] * 4u) : 0.f;
    }
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int i = i0 + kWave * t + lane;
      if (i < nc) ck[i] = __float_as_uint(kv[t]);
    }
  }
  int need = info.need;
  const uint32_t T = resolve_threshold(ck, nc, (int)info.b1, &need, hist);
  // ---- chosen flag of each candidate (bit 31 of its index), lowest index
  // first among keys == T
  int eqs = 0;
  for (int base = 0; base < nc; base += kWave) {
    const int i = base + lane;
    const bool in = i < nc;
    const uint32_t u = in ? ck[i] : 0u;
    const bool eq = in && u == T;
    const uint64_t beq = __ballot(eq);
    const bool take = (in && u > T) || (eq && eqs + (int)lanemask_lt_count(beq) < need);
    if (in && take) ci[i] |= (int)0x80000000u;
    eqs += __builtin_popcountll(beq);
  }
  // ---- emit in ascending order: per word, the above bits and the chosen
  // candidates; the running candidate position finds each candidate's flag
  int out = 0, cpos = 0;
  for (int w0 = 0; w0 < nwords; w0 += kW * kWave) {
    uint32_t aw[kW], cw[kW];
#pragma unroll
    for (int q = 0; q < kW; ++q) {
      const int w = w0 + kW * lane + q;
      aw[q] = w < nwords ? ld_coh_u(bits + word_off(w, 0)) : 0u;
      cw[q] = w < nwords ? ld_coh_u(bits + word_off(w, 1)) : 0u;
    }
    int ccnt = 0;
#pragma unroll
    for (int q = 0; q < kW; ++q) ccnt += __builtin_popcount(cw[q]);
    int ctot;
    int cp = cpos + wave_excl_scan(ccnt, &ctot);
    int ocnt = 0;
#pragma unroll
    for (int q = 0; q < kW; ++q) {
      uint32_t m = cw[q], chosen = 0;
      while (m) {
        const int b = __builtin_ctz(m);
        m &= m - 1;
        if (cp < kFastCap && ci[cp] < 0) chosen |= 1u << b;
        ++cp;
      }
      aw[q] |= chosen;
      ocnt += __builtin_popcount(aw[q]);
    }
    int otot;
    int op = out + wave_excl_scan(ocnt, &otot);
#pragma unroll
    for (int q = 0; q < kW; ++q) {
      uint32_t m = aw[q];
      const int w = w0 + kW * lane + q;
      while (m) {
        const int b = __builtin_ctz(m);
        m &= m - 1;
        if (op < K) sel[op] = 32 * w + b;   // never past the K slots of this row
        ++op;
      }
    }
    out += otot;
    cpos += ctot;
  }
}

// Top-K of one score row whose threshold bin holds more than kFastCap keys
// (the row was written in this launch by other waves: coherent loads).
// ghist: the row's top-digit histogram, cleared here after use.
// path_ctr[1..2]: selections that collected the threshold bin's keys, and
// selections that made two global passes (diagnostic counts, one atomic per
// selection).
__device__ SSPEC_TASK void select_wave(const float* srow, int L, int K, uint32_t* ghist, int32_t* sel, char* wlds,
                                       uint32_t* path_ctr) {
  const int lane = (int)lane_id();
  int* hist = reinterpret_cast<int*>(wlds + SelectWaveLds::kHistOff);
  uint32_t* cand = reinterpret_cast<uint32_t*>(wlds + SelectWaveLds::kCandOff);
  srow = wave_uniform(srow);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(srow, (uint32_t)L * 4u);

  // ---- digit 1 (bits 30..20): from the global histogram, which is reset
  {
    ghist = wave_uniform(ghist);
    const __amdgpu_buffer_rsrc_t rh = make_rsrc(ghist, kHistBins * 4u);
    u32x4 v[kHistBins / kWave / 4];
#pragma unroll
    for (int b = 0; b < kHistBins / kWave / 4; ++b) v[b] = ld_coh4u(rh, (uint32_t)(kHistBins / kWave * lane + 4 * b) * 4u);
#pragma unroll
    for (int b = 0; b < kHistBins / kWave / 4; ++b) {
      const int bin = kHistBins / kWave * lane + 4 * b;
      *reinterpret_cast<u32x4*>(hist + bin) = v[b];
      st_coh4(reinterpret_cast<float*>(ghist + bin), f32x4{0.f, 0.f, 0.f, 0.f});
    }
  }
  if (K <= 0) return;
  int b1, above;
  hist_find(hist, kHistBins, K, b1, above);
  int need = K - above;
  const int n1 = hist[b1];
  int b2, b3;
  const int path = n1 <= kCandCap ? 1 : 2;
  if (lane == 0) __hip_atomic_fetch_add(path_ctr + path, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (path == 1) {
    // ---- collect the keys of bin b1
    int nc = 0;
    for (int j0 = 0; j0 < L; j0 += 4 * kWave * kGroups) {
      u32x4 u[kGroups];
#pragma unroll
      for (int cc = 0; cc < kGroups; ++cc) u[cc] = ld_coh4u(rs, (uint32_t)(j0 + 256 * cc + 4 * lane) * 4u);
#pragma unroll
      for (int cc = 0; cc < kGroups; ++cc)
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
  for (int j0 = 0; j0 < L && out < K; j0 += 4 * kWave * kGroups) {
    u32x4 u[kGroups];
#pragma unroll
    for (int cc = 0; cc < kGroups; ++cc) u[cc] = ld_coh4u(rs, (uint32_t)(j0 + 256 * cc + 4 * lane) * 4u);
#pragma unroll
    for (int cc = 0; cc < kGroups; ++cc) {
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

// Sampled lower bound of a row's k-th largest routing score, shared by the
// routing kernels (clsa_route.hip, clsa_prefill.hip): the sample rank, the
// decode-row sampling plan and the ranking of the sampled key prefixes.
#pragma once

#include "clsa_common.h"

namespace clsa {

// ------------------------------------------------ sampled lower bound of the k-th score
// inverse of score_key
CLSA_DEV float key_to_float(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

// rank among ns regularly spaced samples of a row of n keys whose score
// bounds the row's k-th largest from below with high probability: the
// smallest rho with rho - 4 sqrt(rho) >= k ns / n (a four-sigma margin on
// the number of samples above the k-th largest score).  Larger than ns
// when the sample is too small to bound anything.
CLSA_DEV int sample_rank(int64_t n, int64_t k, int ns) {
  const float kappa = (float)k * (float)ns / (float)n;
  const float sr = 2.0f + sqrtf(4.0f + kappa);
  return (int)ceilf(sr * sr);
}

// Candidate segments of the decode-row filter: a row owns C x segcap
// entries, shared evenly by its cv visible chunks (chunk c's segment starts
// at c x the share); a chunk never holds more candidates than its CH keys.
CLSA_DEV uint32_t row_seg_cap(int C, int segcap, int CH, int64_t cv) {
  const int64_t c = (int64_t)C * segcap / (cv < 1 ? 1 : cv);
  return (uint32_t)(c < CH ? c : CH);
}

// Samples per row of the decode-row threshold estimate (at most), and at
// most how many of each 64 consecutive samples' largest key prefixes are
// kept.
constexpr int kRowSamples = 4096;
constexpr int kRowTop = 16;

// rho-th largest 16-bit key among those held by one wave, exactly: entry u
// of v[] counts where valid(u) holds in its lane (rho at most their number).
// One 1024-bin histogram spanning the keys' actual range, then the <= 64 key
// values of the boundary bin.  h: 1024 words of LDS used by this wave alone.
template <int NPL, class Valid>
CLSA_DEV uint32_t wave_kth_u16(const uint32_t (&v)[NPL], Valid valid, uint32_t rho, uint32_t* h) {
  constexpr int kBins = 1024;
  const int lane = lane_id();
  uint32_t lo = 0xffffu, hi = 0u;
#pragma unroll
  for (int u = 0; u < NPL; ++u)
    if (valid(u)) {
      lo = v[u] < lo ? v[u] : lo;
      hi = v[u] > hi ? v[u] : hi;
    }
  lo = wave_min_u32(lo);
  hi = wave_max_u32(hi);
  const uint32_t range = hi - lo;
  const int shift = range < kBins ? 0 : (32 - __clz(range)) - 10;
#pragma unroll
  for (int i = 0; i < kBins / kWave; ++i) h[lane + kWave * i] = 0u;
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int u = 0; u < NPL; ++u)
    if (valid(u)) atomicAdd(&h[(v[u] - lo) >> shift], 1u);
  __builtin_amdgcn_wave_barrier();
  // bins in descending order: lane l holds bins 1023-16l .. 1008-16l
  uint32_t c[kBins / kWave], sum = 0;
#pragma unroll
  for (int i = 0; i < kBins / kWave; ++i) {
    c[i] = h[kBins - 1 - (kBins / kWave) * lane - i];
    sum += c[i];
  }
  const uint32_t incl = wave_incl_scan(sum);
  const bool mine = incl - sum < rho && rho <= incl;
  uint32_t bin = 0, rin = 0;  // bin of the rho-th largest, its rank inside
  if (mine) {
    uint32_t acc = incl - sum;
#pragma unroll
    for (int i = 0; i < kBins / kWave; ++i) {
      if (acc + c[i] >= rho) {
        bin = kBins - 1 - (kBins / kWave) * lane - i;
        rin = rho - acc;
        break;
      }
      acc += c[i];
    }
  }
  const int src = __ffsll((unsigned long long)__ballot(mine)) - 1;
  bin = __builtin_amdgcn_readlane(bin, src);
  rin = __builtin_amdgcn_readlane(rin, src);
  uint32_t kth = lo + (bin << shift);
  if (shift > 0) {
    // the bin's 2^shift (<= 64) key values, counted exactly
    __builtin_amdgcn_wave_barrier();
    h[lane] = 0u;
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int u = 0; u < NPL; ++u)
      if (valid(u) && (v[u] - kth) < (1u << shift)) atomicAdd(&h[v[u] - kth], 1u);
    __builtin_amdgcn_wave_barrier();
    const uint32_t cc = lane < (1 << shift) ? h[(1 << shift) - 1 - lane] : 0u;  // descending
    const uint32_t inc2 = wave_incl_scan(cc);
    const bool mine2 = inc2 - cc < rin && rin <= inc2;
    const int src2 = __ffsll((unsigned long long)__ballot(mine2)) - 1;
    kth += (uint32_t)((1 << shift) - 1 - src2);
  }
  __builtin_amdgcn_wave_barrier();
  return kth;
}

// Sampling plan of a decode row (one query whose keys no other row shares):
// ns = min(n_vis, kRowSamples) samples, sample i at floor(i n_vis / ns);
// rho from sample_rank; and whether only the top = 8 (or 16, when rho needs
// them) largest key prefixes of each 64 consecutive samples are kept
// (compact: rho well inside their number) or every sample.  Ranking every
// sample takes one wave 8 us at 32K keys (4096 LDS atomics into a
// histogram whose middle bins collide), 16 per 64 samples about 1 us.
struct RowPlan {
  int ns, rho, top, nkept;
  bool compact;
};
CLSA_DEV RowPlan row_plan(int64_t n_vis, int64_t k_eff) {
  RowPlan p;
  p.ns = (int)(n_vis < kRowSamples ? n_vis : kRowSamples);
  p.rho = sample_rank(n_vis, k_eff, p.ns);
  const int waves = (p.ns + kWave - 1) / kWave;
  p.top = 2 * p.rho <= waves * 8 ? 8 : kRowTop;
  p.nkept = waves * p.top;
  p.compact = 2 * p.rho <= p.nkept;
  return p;
}

// One wave: a decode row's filter threshold from the prefixes its sampling
// pass stored at `row` (rho <= ns): the rho-th largest of them as the
// smallest float with that prefix.  With compact lists this is at most the
// rho-th largest sample (the kept prefixes are some of the samples), so it
// is a lower bound of the sample's rho-th score either way.  h: 1024 words
// of LDS for this wave.
// compact lists: lane l holds wave l's kept entries top l .. top l + top - 1
// in v[0 .. top) (zeros past the list)
CLSA_DEV void load_row_kept(const uint16_t* row, const RowPlan& p, uint32_t (&v)[kRowTop]) {
  static_assert(kRowTop == 16, "at most two 16-byte loads per lane");
  const int lane = lane_id();
  const int last = p.nkept / p.top - 1;  // lanes past the list re-read its last entries
  const u32x4_t* src = reinterpret_cast<const u32x4_t*>(row + (lane < last ? lane : last) * p.top);
  const u32x4_t x0 = src[0];
  const u32x4_t x1 = src[p.top / 8 - 1];  // the same 16 bytes again when top = 8
  const bool ok = lane <= last;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    v[e] = ok ? (x0[e / 2] >> (16 * (e & 1))) & 0xffffu : 0u;
    v[8 + e] = ok && p.top > 8 ? (x1[e / 2] >> (16 * (e & 1))) & 0xffffu : 0u;
  }
}
CLSA_DEV float rank_row_kept(const uint32_t (&v)[kRowTop], const RowPlan& p, uint32_t* h) {
  const bool ok = p.top * lane_id() < p.nkept;
  const int top = p.top;
  return key_to_float(
      wave_kth_u16(v, [&](int u) { return ok && u < top; }, (uint32_t)p.rho, h) << 16);
}

CLSA_DEV float rank_row_samples(const uint16_t* row, const RowPlan& p, uint32_t* h) {
  const int lane = lane_id();
  const u32x4_t* sp = reinterpret_cast<const u32x4_t*>(row);
  uint32_t kth;
  if (p.compact) {
    uint32_t v[kRowTop];
    load_row_kept(row, p, v);
    return rank_row_kept(v, p, h);
  } else {
    // every sample: lane l holds samples 512 u + 8 l + e in v[8 u + e]
    uint32_t v[kRowSamples / kWave];
#pragma unroll
    for (int u = 0; u < kRowSamples / (8 * kWave); ++u) {
      const int i0 = u * 8 * kWave + 8 * lane;
      const u32x4_t x = i0 < p.ns ? sp[u * kWave + lane] : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
      for (int e = 0; e < 8; ++e) v[8 * u + e] = (x[e / 2] >> (16 * (e & 1))) & 0xffffu;
    }
    kth = wave_kth_u16(
        v, [&](int u) { return (u / 8) * 8 * kWave + 8 * lane + (u % 8) < p.ns; }, (uint32_t)p.rho, h);
  }
  return key_to_float(kth << 16);
}

}  // namespace clsa

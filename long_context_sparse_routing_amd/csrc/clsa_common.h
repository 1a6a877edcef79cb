// Device-side helpers shared by the libclsa kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/clsa.h"

#define CLSA_DEV __device__ __forceinline__

namespace clsa {

constexpr int kWave = 64;

// ------------------------------------------------------------ vector loads
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte load with the non-temporal (streaming) hint, for data read once:
// gathered K/V rows and the routing-key scan.
CLSA_DEV u32x4_t load_stream16(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}

// ---------------------------------------------------------------- bfloat16
CLSA_DEV float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
CLSA_DEV float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float -> bfloat16 with round-to-nearest-even; NaN stays a (quiet) NaN.
CLSA_DEV uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// c + a.lo * b.lo + a.hi * b.hi over two packed bf16 pairs (v_dot2_f32_bf16)
CLSA_DEV float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// ------------------------------------------------------- order-preserving key
// Monotone map float -> uint32: a > b  <=>  key(a) > key(b), and -0.0 maps to
// the key of +0.0 so the two compare equal (as they do as floats).
CLSA_DEV uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---------------------------------------------------------------- wave ops
CLSA_DEV int lane_id() { return (int)__lane_id(); }

// number of set bits of `mask` in lanes below this one
CLSA_DEV uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

CLSA_DEV float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}
CLSA_DEV float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}
// DPP lane move: the value of another lane of v, per the DPP control word,
// or `old` where the source lane is out of range or the row is masked off.
// No LDS round trip, unlike a shuffle.
template <int CTRL, int ROW_MASK>
CLSA_DEV uint32_t dpp_move(uint32_t old, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, ROW_MASK, 0xf, false);
}
constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;
constexpr int kRowBcast15 = 0x142, kRowBcast31 = 0x143;

// inclusive scan across the wave with an associative, commutative op whose
// identity is `id`: Hillis-Steele within each 16-lane row (row shifts by 1,
// 2, 4, 8), then the row totals broadcast into the rows above them
template <class Op>
CLSA_DEV uint32_t wave_scan_dpp(uint32_t v, uint32_t id, Op op) {
  v = op(v, dpp_move<kRowShr1, 0xf>(id, v));
  v = op(v, dpp_move<kRowShr2, 0xf>(id, v));
  v = op(v, dpp_move<kRowShr4, 0xf>(id, v));
  v = op(v, dpp_move<kRowShr8, 0xf>(id, v));
  v = op(v, dpp_move<kRowBcast15, 0xa>(id, v));  // row 0 total into row 1, row 2 into row 3
  v = op(v, dpp_move<kRowBcast31, 0xc>(id, v));  // rows 0-1 total into rows 2 and 3
  return v;
}

// inclusive prefix sum across the wave
CLSA_DEV uint32_t wave_incl_scan(uint32_t v) {
  return wave_scan_dpp(v, 0u, [](uint32_t x, uint32_t y) { return x + y; });
}
// totals over the wave (wave-uniform results)
CLSA_DEV uint32_t wave_sum_u32(uint32_t v) {
  return __builtin_amdgcn_readlane(wave_incl_scan(v), kWave - 1);
}
CLSA_DEV uint32_t wave_min_u32(uint32_t v) {
  return __builtin_amdgcn_readlane(
      wave_scan_dpp(v, 0xffffffffu, [](uint32_t x, uint32_t y) { return x < y ? x : y; }), kWave - 1);
}
CLSA_DEV uint32_t wave_max_u32(uint32_t v) {
  return __builtin_amdgcn_readlane(
      wave_scan_dpp(v, 0u, [](uint32_t x, uint32_t y) { return x > y ? x : y; }), kWave - 1);
}

// Block-wide inclusive scan of one value per thread.  `tmp` must hold one
// uint32 per wave.  Every thread of the block must call it.
template <int NT>
CLSA_DEV uint32_t block_incl_scan(uint32_t v, uint32_t* tmp) {
  constexpr int NW = NT / kWave;
  const int w = threadIdx.x / kWave;
  uint32_t inc = wave_incl_scan(v);
  if (lane_id() == kWave - 1) tmp[w] = inc;
  __syncthreads();
  uint32_t add = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i)
    if (i < w) add += tmp[i];
  __syncthreads();
  return inc + add;
}

// Ordered compaction of one NT-element slice: returns this thread's slot
// among the set predicates of the slice (ascending thread order) and the
// slice's total in *total.  `wcnt` holds one uint32 per wave; every thread
// of the block must call it.
template <int NT = 256>
CLSA_DEV uint32_t block_rank(bool p, uint32_t* wcnt, uint32_t* total) {
  const int w = threadIdx.x / kWave;
  const uint64_t mask = __ballot(p);
  if (lane_id() == 0) wcnt[w] = (uint32_t)__popcll(mask);
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NT / kWave; ++i) {
    before += (i < w) ? wcnt[i] : 0u;
    tot += wcnt[i];
  }
  __syncthreads();
  *total = tot;
  return before + lanes_below(mask);
}

__host__ __device__ inline int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }

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

// Host helpers implemented in clsa_api.hip.
namespace clsa {
// Zero `bytes` (multiple of 4) at `p` with a fill kernel on `stream`.
hipError_t zero_fill(void* p, size_t bytes, hipStream_t stream);
inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
}  // namespace clsa

// Block-wide exact selection helpers shared by the select kernels of the
// routing paths (512-thread workgroups): the bin of a rank in a histogram,
// and the exact rank-th largest of keys held in registers.
#pragma once

#include "clsa_common.h"

namespace clsa {

constexpr int kSelNT = 512;  // threads of every workgroup that calls these

// ----------------------------------------------------- LDS radix helpers
// Bin holding the rank-th largest element of histogram h[0..NB) (bin NB-1
// holds the largest values); rank is 1-based.  out2 = {bin, rank within}.
template <int NB>
CLSA_DEV void find_bin_desc(const uint32_t* h, uint32_t rank, uint32_t* tmp, uint32_t* out2) {
  constexpr int PER = NB / kSelNT;
  const int tid = threadIdx.x;
  uint32_t v[PER], sum = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    v[i] = h[NB - 1 - PER * tid - i];
    sum += v[i];
  }
  const uint32_t incl = block_incl_scan<kSelNT>(sum, tmp);
  const uint32_t excl = incl - sum;
  if (excl < rank && rank <= incl) {
    uint32_t acc = excl;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (acc + v[i] >= rank) {
        out2[0] = (uint32_t)(NB - 1 - PER * tid - i);
        out2[1] = rank - acc;
        break;
      }
      acc += v[i];
    }
  }
  __syncthreads();
}

constexpr int kSmall = 256;  // boundary-bin elements ranked pairwise

struct SelScratch {  // LDS scratch of the block selects
  uint32_t h[2048];
  uint32_t small[kSmall];
  uint32_t tmp[kSelNT / kWave];
  uint32_t lo[kSelNT / kWave], hi[kSelNT / kWave];
  uint32_t bc[8];
};

// Exact rank-th largest of the keys held in registers, 1 <= rank <= the
// number of valid keys: thread t holds k[0 .. cnt) (cnt <= NPER).  One pass
// of a 2048-bin histogram spanning the keys' actual range; the boundary bin
// is ranked pairwise when it holds at most kSmall keys, and refined by
// further 11-bit passes otherwise (massive ties).  *left gets how many keys
// equal to the result are needed to reach the rank, *eq_total how many
// there are.
template <int NPER>
CLSA_DEV uint32_t kth_regs(const uint32_t (&k)[NPER], int cnt, uint32_t rank, SelScratch& S,
                           uint32_t* left, uint32_t* eq_total) {
  const int tid = threadIdx.x, w = tid / kWave;
  // the first pass's histogram and compaction counter are cleared before the
  // barrier that publishes the range
  for (int i = tid; i < 2048; i += kSelNT) S.h[i] = 0u;
  if (tid == 0) S.bc[2] = 0u;
  uint32_t lo = 0xffffffffu, hi = 0u;
#pragma unroll
  for (int u = 0; u < NPER; ++u)
    if (u < cnt) {
      lo = k[u] < lo ? k[u] : lo;
      hi = k[u] > hi ? k[u] : hi;
    }
  lo = wave_min_u32(lo);
  hi = wave_max_u32(hi);
  if (lane_id() == 0) S.lo[w] = lo, S.hi[w] = hi;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kSelNT / kWave; ++i) {
    lo = S.lo[i] < lo ? S.lo[i] : lo;
    hi = S.hi[i] > hi ? S.hi[i] : hi;
  }
  const uint32_t range = hi - lo;
  int shift = range < 2048u ? 0 : (32 - __clz(range)) - 11;
  int shift_prev = 32;
  uint32_t prefix = 0;  // (key - lo) >> shift_prev of the keys still in play
  for (bool first = true;; first = false) {
    if (!first) {
      for (int i = tid; i < 2048; i += kSelNT) S.h[i] = 0u;
      if (tid == 0) S.bc[2] = 0u;
      __syncthreads();
    }
#pragma unroll
    for (int u = 0; u < NPER; ++u)
      if (u < cnt) {
        const uint32_t d = k[u] - lo;
        if (shift_prev >= 32) atomicAdd(&S.h[d >> shift], 1u);
        else if ((d >> shift_prev) == prefix)
          atomicAdd(&S.h[(d >> shift) - (prefix << (shift_prev - shift))], 1u);
      }
    __syncthreads();
    find_bin_desc<2048>(S.h, rank, S.tmp, S.bc);
    const uint32_t bin = S.bc[0], r = S.bc[1], c = S.h[bin];
    const uint32_t full = (shift_prev >= 32 ? 0u : prefix << (shift_prev - shift)) + bin;
    if (shift == 0) {
      *left = r;
      *eq_total = c;
      __syncthreads();
      return lo + full;
    }
    if (c <= (uint32_t)kSmall) {
#pragma unroll
      for (int u = 0; u < NPER; ++u)
        if (u < cnt && ((k[u] - lo) >> shift) == full) S.small[atomicAdd(&S.bc[2], 1u)] = k[u];
      __syncthreads();
      for (uint32_t e = tid; e < c; e += kSelNT) {
        const uint32_t v = S.small[e];
        uint32_t gt = 0, eq = 0;
        for (uint32_t f = 0; f < c; ++f) {
          gt += S.small[f] > v ? 1u : 0u;
          eq += S.small[f] == v ? 1u : 0u;
        }
        if (gt < r && r <= gt + eq) {  // equal keys all write the same values
          S.bc[3] = v;
          S.bc[4] = r - gt;
          S.bc[5] = eq;
        }
      }
      __syncthreads();
      const uint32_t kth = S.bc[3];
      *left = S.bc[4];
      *eq_total = S.bc[5];
      __syncthreads();
      return kth;
    }
    rank = r;
    prefix = full;
    shift_prev = shift;
    shift = shift > 11 ? shift - 11 : 0;
    __syncthreads();
  }
}


// LDS of a select's position bitmap: wpt words per thread, followed by one
// 16-bit prefix per word (the marks before it; a select marks at most the
// candidates it holds, far below 65536).
__host__ __device__ inline size_t select_bitmap_lds_bytes(int64_t wpt) {
  return (size_t)wpt * kSelNT * (sizeof(uint32_t) + sizeof(uint16_t));
}

// The k_eff largest of the keys held in registers (thread t: key[u], pos[u]
// for u < cnt; positions distinct), written to out[0 .. k_eff) in ascending
// position order; equal keys at the boundary are taken in position order.
// bitmap4: zeroed LDS bitmap over positions, wpt words per thread (a
// multiple of 4), then room for the word prefixes (select_bitmap_lds_bytes).
// Every thread of the block calls it.
template <int NPER>
CLSA_DEV void select_emit(const uint32_t (&key)[NPER], const uint32_t (&pos)[NPER], int cnt,
                          uint32_t k_eff, SelScratch& S, u32x4_t* bitmap4, int wpt, int32_t* out) {
  uint32_t* bitmap = reinterpret_cast<uint32_t*>(bitmap4);
  const int tid = threadIdx.x;
  const int w0 = tid * wpt;
  uint32_t left, eq_total;
  const uint32_t kstar = kth_regs<NPER>(key, cnt, k_eff, S, &left, &eq_total);

  // mark the selection: keys above kstar, and of the keys equal to it the
  // `left` lowest positions
  if (left == eq_total) {
#pragma unroll
    for (int u = 0; u < NPER; ++u)
      if (u < cnt && key[u] >= kstar) atomicOr(&bitmap[pos[u] >> 5], 1u << (pos[u] & 31));
  } else if (eq_total <= (uint32_t)kSmall) {
    if (tid == 0) S.bc[2] = 0u;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < NPER; ++u)
      if (u < cnt && key[u] == kstar) S.small[atomicAdd(&S.bc[2], 1u)] = pos[u];
    __syncthreads();
    for (uint32_t e = tid; e < eq_total; e += kSelNT) {
      const uint32_t p = S.small[e];
      uint32_t lower = 0;
      for (uint32_t f = 0; f < eq_total; ++f) lower += S.small[f] < p ? 1u : 0u;
      if (lower < left) atomicOr(&bitmap[p >> 5], 1u << (p & 31));
    }
#pragma unroll
    for (int u = 0; u < NPER; ++u)
      if (u < cnt && key[u] > kstar) atomicOr(&bitmap[pos[u] >> 5], 1u << (pos[u] & 31));
  } else {
    // massive ties: mark every equal key, keep the first `left` in position
    // order, then add the keys above kstar
#pragma unroll
    for (int u = 0; u < NPER; ++u)
      if (u < cnt && key[u] == kstar) atomicOr(&bitmap[pos[u] >> 5], 1u << (pos[u] & 31));
    __syncthreads();
    uint32_t mine = 0;
    for (int i = w0; i < w0 + wpt; ++i) mine += __popc(bitmap[i]);
    uint32_t rank = block_incl_scan<kSelNT>(mine, S.tmp) - mine;
    for (int i = w0; i < w0 + wpt; ++i) {
      uint32_t word = bitmap[i];
      for (uint32_t rest = word; rest != 0u; rest &= rest - 1u) {
        if (rank >= left) word &= ~(rest & (0u - rest));
        ++rank;
      }
      bitmap[i] = word;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < NPER; ++u)
      if (u < cnt && key[u] > kstar) atomicOr(&bitmap[pos[u] >> 5], 1u << (pos[u] & 31));
  }
  __syncthreads();

  // emit in position order: the output slot of a selected position is the
  // number of marked positions below it -- the prefix of its bitmap word,
  // then a popcount inside the word -- so every thread writes its own
  // selected candidates independently
  uint2* wpre2 = reinterpret_cast<uint2*>(bitmap + (size_t)wpt * kSelNT);  // 4 prefixes each
  uint32_t mine = 0;
  for (int i = w0; i < w0 + wpt; i += 4) {
    const u32x4_t x = bitmap4[i / 4];
    mine += __popc(x[0]) + __popc(x[1]) + __popc(x[2]) + __popc(x[3]);
  }
  uint32_t run = block_incl_scan<kSelNT>(mine, S.tmp) - mine;
  for (int i = w0; i < w0 + wpt; i += 4) {
    const u32x4_t x = bitmap4[i / 4];
    const uint32_t r1 = run + __popc(x[0]), r2 = r1 + __popc(x[1]), r3 = r2 + __popc(x[2]);
    wpre2[i / 4] = make_uint2(run | (r1 << 16), r2 | (r3 << 16));
    run = r3 + __popc(x[3]);
  }
  __syncthreads();
  const uint16_t* wpre = reinterpret_cast<const uint16_t*>(wpre2);
#pragma unroll
  for (int u = 0; u < NPER; ++u) {
    if (u < cnt) {
      const uint32_t p = pos[u];
      const uint32_t word = bitmap[p >> 5];
      if ((word >> (p & 31u)) & 1u)
        out[wpre[p >> 5] + __popc(word & ((1u << (p & 31u)) - 1u))] = (int32_t)p;
    }
  }
}

}  // namespace clsa

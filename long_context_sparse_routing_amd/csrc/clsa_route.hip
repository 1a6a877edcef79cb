// Routing for shared-routing sparse attention: one score pass over all
// visible routing keys, then an exact top-k (or half-space) selection that
// emits each row's key positions in ascending order.
//
// Method: CLSA explainer (ai-papers.net), section "CLSAの仕組み" -- a single
// routing step picks the top-k KV positions for each query token and every
// cross-decoder layer reuses them; section "計算コストの削減効果" -- this is
// paid once per token instead of once per layer.  Threshold mode: Louver
// summary (gist.science, arXiv 2605.06763), section "1. 半空間範囲検索への帰着"
// -- all keys with <q, k> >= tau.
//
// Kernels (grid = chunks x rows; a chunk is CH consecutive keys of a row).
// Workgroups never wait on each other; kernel boundaries order the passes.
//   route_score    s_j = q . K_idx[j] (fp32 accumulation, coalesced 16-byte
//                  loads + a butterfly reduce-scatter across the lanes of a
//                  key row), stores order-preserving uint32 keys, and either
//                  adds the chunk's histogram of the top 11 key bits to the
//                  row's 2048-bucket histogram (top-k) or counts keys >=
//                  key(tau) per chunk (threshold).
//   route_cands    (top-k) finds the bucket T1 holding the k-th largest key
//                  from the histogram, counts keys above T1 per chunk, and
//                  stores the chunk's keys in T1 (ascending position) as
//                  candidates: low 21 key bits, then the inverted position so
//                  that lower positions win ties.
//                  It also histograms key bits 20..10 of those candidates.
//   route_select   (top-k, one workgroup per row) finds the second-level bin
//                  T2 of the k-th largest key from that histogram; each thread
//                  walks its own chunks' candidates once, counting those above
//                  T2 and collecting those in T2 (typically a handful), which
//                  are ranked pairwise (lower position wins ties, through the
//                  composite).  It writes the composite threshold Tc and every
//                  chunk's output offset.
//   route_compact  writes the selected positions of its chunk in ascending
//                  order with wave ballots from the chunk's offset; pads
//                  with -1 and sets counts.
// bf16 top-k with k <= 2048 over at most 512K keys takes a shorter path
// instead: row_sample (clsa_prefill.hip) scores up to 4096 evenly spaced
// keys of each row; route_score in filter mode ranks them (every workgroup
// for itself) for a lower bound T of the row's k-th largest score and
// appends the chunk's keys scoring >= T as (position, score) to the row's
// candidate list;
// block_select (clsa_prefill.hip) takes the exact top-k of those candidates.
// Scores are the same in both paths.
#include <mutex>

#include "clsa_common.h"
#include "clsa_rowplan.h"

namespace clsa {

namespace {

constexpr int kNT = 256;          // threads per workgroup
constexpr int kBuckets = 2048;    // histogram of the top 11 key bits
constexpr int kBucketShift = 21;
constexpr uint32_t kLowMask = (1u << kBucketShift) - 1u;
constexpr int kMaxChunks = 4096;  // chunks per row
constexpr int kMaxFilterCH = 2048;  // keys per chunk in filter mode (at most)
constexpr int kMaxHeads = 64;       // index heads of an aggregated routing call

// what route_score does with the scores
constexpr int kHist = 0;    // top-k: keys + histogram of the top 11 bits
constexpr int kCount = 1;   // threshold: keys + count of keys >= tau per chunk
constexpr int kFilter = 2;  // top-k: candidates >= thr[r] into the chunk's segment

struct RouteArgs {
  const void* q;          // [R][d]
  const void* K;          // [B][n_cap][d]
  const int32_t* n_ctx;   // [B] or null
  const float* tau;       // [R] (threshold mode)
  int32_t* idx;           // [R][cap]
  int32_t* counts;        // [R]
  int64_t n_cap;
  int64_t q_pos0;
  int B, M, k, cap;
  int CH, C;              // keys per chunk, chunks per row (max)
  // workspace
  uint32_t* ghist;        // [R][2048]   top 11 key bits (zeroed at the start of each call)
  uint32_t* ghist2;       // [R][2048]   key bits 20..10 of the keys in bucket T1 (zeroed too)
  uint32_t* rowsel;       // [R][4]      T1, r1, Tc (64-bit)
  uint32_t* off;          // [R][C]      output offset of each chunk (top-k)
  uint32_t* cgt;          // [R][C]      keys above T1 / keys >= tau, per chunk
  uint32_t* ccnt;         // [R][C]      candidates per chunk
  uint32_t* keys;         // [R][n_cap]
  uint64_t* cand;         // [R][n_cap]  chunk c's candidates at [c*CH, ...)
  // filter mode
  const uint16_t* samp;   // [R][kRowSamples] sampled key prefixes (row_sample)
  uint32_t* segcnt;       // [R][C]     candidates found per chunk (true count)
  uint64_t* seg;          // [R][C * segcap] position | score bits << 32, per chunk
  int segcap;             // entries per chunk and row (shared by visible chunks)
  // cross-layer aggregation (exhaustive path): heads 1 .. H-1 beyond (q, K),
  // whose scores are added to head 0's before the selection
  const void* qh[kMaxHeads];
  const void* Kh[kMaxHeads];
  int H;
};

CLSA_DEV int64_t visible(const RouteArgs& a, int r) {
  const int b = r / a.M, m = r % a.M;
  int64_t n = a.n_ctx ? (int64_t)a.n_ctx[b] : a.n_cap;
  n = n < 0 ? 0 : (n > a.n_cap ? a.n_cap : n);
  if (a.q_pos0 >= 0) {
    const int64_t lim = a.q_pos0 + m + 1;
    n = n < lim ? n : lim;
  }
  return n;
}

CLSA_DEV int64_t chunks_of(int64_t n_vis, int CH) {
  const int64_t c = ceil_div64(n_vis, CH);
  return c < 1 ? 1 : c;
}

CLSA_DEV uint64_t composite(uint32_t key, uint32_t j) {
  return ((uint64_t)(key & kLowMask) << 32) | (uint64_t)(~j);
}

// --------------------------------------------------------------- dot pieces
template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int kPer16 = 4;
  CLSA_DEV static float dot(const u32x4_t v, const float* qf) {
    float s = qf[0] * __uint_as_float(v[0]);
    s = fmaf(qf[1], __uint_as_float(v[1]), s);
    s = fmaf(qf[2], __uint_as_float(v[2]), s);
    s = fmaf(qf[3], __uint_as_float(v[3]), s);
    return s;
  }
  CLSA_DEV static void load_q(const void* q, size_t off, float* qf) {
    const float* p = static_cast<const float*>(q) + off;
#pragma unroll
    for (int e = 0; e < 4; ++e) qf[e] = p[e];
  }
};
template <> struct Elem<uint16_t> {
  static constexpr int kPer16 = 8;
  CLSA_DEV static float dot(const u32x4_t v, const float* qf) {
    // bf16 x bf16 products are exact in fp32, so fma and mul+add agree.
    float s = qf[0] * bf16_lo(v[0]);
    s = fmaf(qf[1], bf16_hi(v[0]), s);
    s = fmaf(qf[2], bf16_lo(v[1]), s);
    s = fmaf(qf[3], bf16_hi(v[1]), s);
    s = fmaf(qf[4], bf16_lo(v[2]), s);
    s = fmaf(qf[5], bf16_hi(v[2]), s);
    s = fmaf(qf[6], bf16_lo(v[3]), s);
    s = fmaf(qf[7], bf16_hi(v[3]), s);
    return s;
  }
  CLSA_DEV static void load_q(const void* q, size_t off, float* qf) {
    const uint16_t* p = static_cast<const uint16_t*>(q) + off;
#pragma unroll
    for (int e = 0; e < 8; ++e) qf[e] = __uint_as_float((uint32_t)p[e] << 16);
  }
};

// The value of lane (lane ^ M): DPP moves within a 16-lane row for M <= 8
// (quad permutes for 1 and 2, row shifts for 4 and 8), no LDS round trip.
template <int M>
CLSA_DEV float lane_xor(float v, int lane) {
  const int x = __float_as_int(v);
  if constexpr (M == 1) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0xB1, 0xf, 0xf, false));  // [1,0,3,2]
  } else if constexpr (M == 2) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x4E, 0xf, 0xf, false));  // [2,3,0,1]
  } else if constexpr (M == 4 || M == 8) {
    const int up = __builtin_amdgcn_update_dpp(0, x, 0x110 + M, 0xf, 0xf, false);  // row_shr: lane - M
    const int dn = __builtin_amdgcn_update_dpp(0, x, 0x100 + M, 0xf, 0xf, false);  // row_shl: lane + M
    return __int_as_float((lane & M) ? up : dn);
  } else {
    return __shfl_xor(v, M);
  }
}

// U partial sums per lane, U consecutive lanes per key row.  After the
// butterfly, the lane with in-group position p holds the full sum of partial
// index p.  The addition tree is the same for every partial index, so
// identical key rows give bit-identical scores.
template <int U, int M = U / 2>
CLSA_DEV void reduce_scatter_step(float (&v)[U], int lane) {
  if constexpr (M >= 1) {
    const bool up = (lane & M) != 0;
#pragma unroll
    for (int i = 0; i < M; ++i) {
      const float send = up ? v[i] : v[i + M];
      const float keep = up ? v[i + M] : v[i];
      v[i] = keep + lane_xor<M>(send, lane);
    }
    reduce_scatter_step<U, M / 2>(v, lane);
  }
}
template <int U>
CLSA_DEV float reduce_scatter(float (&v)[U], int lane) {
  reduce_scatter_step<U>(v, lane);
  return v[0];
}

// Sum over the first `n` entries of `arr` (global), result in every thread.
CLSA_DEV uint32_t block_sum_prefix(const uint32_t* arr, int64_t n, uint32_t* tmp) {
  uint32_t loc = 0;
  for (int64_t i = threadIdx.x; i < n; i += kNT) loc += arr[i];
  uint32_t tot = wave_sum_u32(loc);
  const int w = threadIdx.x / kWave;
  if (lane_id() == 0) tmp[w] = tot;
  __syncthreads();
  uint32_t s = 0;
#pragma unroll
  for (int i = 0; i < kNT / kWave; ++i) s += tmp[i];
  __syncthreads();
  return s;
}

// ------------------------------------------------------------------- score
template <typename T, int D, int MODE>
__global__ __launch_bounds__(kNT) void route_score(RouteArgs a) {
  constexpr int kEPL = Elem<T>::kPer16;        // elements per 16-byte segment
  constexpr int kLPR = D / kEPL;               // lanes per key row
  constexpr int kKPI = kWave / kLPR;           // key rows per wave load
  constexpr int kU = kLPR;                     // loads per lane per wave pass
  static_assert(kLPR >= 2 && kLPR <= 32, "unsupported row width");
  constexpr bool TOPK = MODE == kHist;

  __shared__ uint32_t hist[TOPK ? kBuckets : 1];
  __shared__ uint32_t tmp[kNT / kWave];
  __shared__ uint64_t cbuf[MODE == kFilter ? kMaxFilterCH : 1];  // the chunk's candidates
  __shared__ uint32_t wh[MODE == kFilter ? 1024 : 1];
  __shared__ uint32_t ccount;
  __shared__ float sthr;

  const int c = blockIdx.x, r = blockIdx.y;
  const int tid = threadIdx.x, lane = lane_id(), w = tid / kWave;
  const int b = r / a.M;
  const int64_t n_vis = visible(a, r);
  const int grp = lane / kLPR, pos = lane % kLPR;
  float qf[kEPL];
  Elem<T>::load_q(a.q, (size_t)r * D + (size_t)pos * kEPL, qf);
  const char* Kb = static_cast<const char*>(a.K) + (size_t)b * a.n_cap * D * sizeof(T);
  const int64_t j0 = (int64_t)c * a.CH;
  u32x4_t v[kU];
  // this wave's keys wbase .. wbase + 63 (rows past n_vis read row 0)
  auto issue = [&](int64_t wbase) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t j = wbase + u * kKPI + grp;
      const int64_t jj = j < n_vis ? j : 0;
      v[u] = load_stream16(Kb + (size_t)jj * D * sizeof(T) + pos * 16);
    }
  };
  bool pre = false;  // the wave's first keys are already in flight
  float thr = 0.f;
  if constexpr (MODE == kFilter) {
    const int64_t k_eff = (int64_t)a.k < n_vis ? (int64_t)a.k : n_vis;
    if (k_eff >= n_vis) return;  // every visible key is selected: no candidates needed
    if (c >= chunks_of(n_vis, a.CH)) return;
    // the row's threshold, ranked from its samples by wave 0 (-inf when
    // the sample is too small to bound the k-th score), while every wave's
    // first keys are already on their way
    const RowPlan p = row_plan(n_vis, k_eff);
    const bool ranks = p.rho <= p.ns;
    const int64_t wb0 = j0 + w * kWave;
    const uint16_t* srow = a.samp + (size_t)r * kRowSamples;
    float t = -INFINITY;
    // The compact list is read first (by every wave: 1 KB, no branch) and
    // the keys after it, pinned in that order, so the ranking waits on the
    // list alone.
    uint32_t sv[kRowTop];
    load_row_kept(srow, p, sv);
    issue(wb0);
    pre = true;
    asm volatile("" ::: "memory");
    if (w == 0 && ranks) t = p.compact ? rank_row_kept(sv, p, wh) : rank_row_samples(srow, p, wh);
    if (w == 0 && lane == 0) {
      sthr = t;
      ccount = 0u;
    }
    // a barrier on LDS alone: the key loads stay in flight
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    thr = sthr;
  }
  if (c >= chunks_of(n_vis, a.CH)) return;
  if (TOPK) {
    if ((int64_t)a.k >= n_vis) return;  // every visible key is selected
    for (int i = tid; i < kBuckets; i += kNT) hist[i] = 0u;
    __syncthreads();
  }
  uint32_t tkey = 0;
  if (MODE == kCount) tkey = score_key(a.tau[r]);

  uint32_t* keys_row = a.keys + (size_t)r * a.n_cap;
  uint32_t n_ge = 0;

  for (int it = 0; it < a.CH / kNT; ++it) {
    const int64_t wbase = j0 + (int64_t)it * kNT + w * kWave;
    if (wbase >= n_vis) break;
    float part[kU];
    if (!(pre && it == 0)) issue(wbase);
#pragma unroll
    for (int u = 0; u < kU; ++u) part[u] = Elem<T>::dot(v[u], qf);
    if constexpr (TOPK) {
      // aggregated heads: each head's partial dot products are added before
      // the lane reduction, so every key sums its heads in the same order
      for (int h = 1; h < a.H; ++h) {
        float qhf[kEPL];
        Elem<T>::load_q(a.qh[h], (size_t)r * D + (size_t)pos * kEPL, qhf);
        const char* Kbh = static_cast<const char*>(a.Kh[h]) + (size_t)b * a.n_cap * D * sizeof(T);
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          const int64_t j = wbase + u * kKPI + grp;
          v[u] = load_stream16(Kbh + (size_t)(j < n_vis ? j : 0) * D * sizeof(T) + pos * 16);
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) part[u] += Elem<T>::dot(v[u], qhf);
      }
    }
    const float s = reduce_scatter<kU>(part, lane);
    const int64_t j = wbase + pos * kKPI + grp;
    if (MODE == kFilter) {
      const bool hit = j < n_vis && s >= thr;
      const uint64_t hm = __ballot(hit);
      if (hm != 0ull) {  // wave-uniform
        uint32_t base = 0;
        if (lane == 0) base = atomicAdd(&ccount, (uint32_t)__popcll(hm));
        base = __builtin_amdgcn_readfirstlane(base);
        if (hit)
          cbuf[base + lanes_below(hm)] =
              ((uint64_t)__float_as_uint(s) << 32) | (uint64_t)(uint32_t)j;
      }
    } else if (j < n_vis) {
      const uint32_t key = score_key(s);
      keys_row[j] = key;
      if (TOPK) atomicAdd(&hist[key >> kBucketShift], 1u);
      else n_ge += (key >= tkey) ? 1u : 0u;
    }
  }

  if (MODE == kFilter) {
    // the chunk's candidates into its own segment of the row, with the true
    // count (entries past the segment are counted, not kept).  No atomics
    // between workgroups: a device-scope reservation on one counter per row
    // cost every workgroup a round trip at its end (scan 26 -> 21 us at
    // 8 rows of 128K keys without it).
    __syncthreads();
    const uint32_t n = ccount;
    const uint32_t cap = row_seg_cap(a.C, a.segcap, a.CH, chunks_of(n_vis, a.CH));
    if (tid == 0) a.segcnt[(size_t)r * a.C + c] = n;
    uint64_t* dst = a.seg + (size_t)r * a.C * a.segcap + (size_t)c * cap;
    const uint32_t m = n < cap ? n : cap;
    for (uint32_t i = tid; i < m; i += kNT) dst[i] = cbuf[i];
  } else if (TOPK) {
    __syncthreads();
    uint32_t* gh = a.ghist + (size_t)r * kBuckets;
    for (int i = tid; i < kBuckets; i += kNT) {
      const uint32_t h = hist[i];
      if (h) atomicAdd(&gh[i], h);
    }
  } else {
    const uint32_t tot = wave_sum_u32(n_ge);
    if (lane == 0) tmp[w] = tot;
    __syncthreads();
    if (tid == 0) {
      uint32_t t = 0;
      for (int i = 0; i < kNT / kWave; ++i) t += tmp[i];
      a.cgt[(size_t)r * a.C + c] = t;
    }
  }
}

// -------------------------------------------------------------- candidates
// Bucket T1 holding the k_eff-th largest key and how many keys r1 to take
// from it.  Thread t owns buckets 2047-8t .. 2040-8t (descending).
CLSA_DEV void find_bucket(const uint32_t* gh, uint32_t k_eff, uint32_t* tmp, uint32_t* out2) {
  const int tid = threadIdx.x;
  uint32_t h[8], sum = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    h[i] = gh[kBuckets - 1 - 8 * tid - i];
    sum += h[i];
  }
  const uint32_t incl = block_incl_scan<kNT>(sum, tmp);
  const uint32_t excl = incl - sum;
  if (excl < k_eff && k_eff <= incl) {
    uint32_t acc = excl;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (acc + h[i] >= k_eff) {
        out2[0] = (uint32_t)(kBuckets - 1 - 8 * tid - i);
        out2[1] = k_eff - acc;
        break;
      }
      acc += h[i];
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(kNT) void route_cands(RouteArgs a) {
  __shared__ uint32_t tmp[kNT / kWave];
  __shared__ uint32_t wcnt[kNT / kWave];
  __shared__ uint32_t sel[2];

  const int c = blockIdx.x, r = blockIdx.y;
  const int tid = threadIdx.x, lane = lane_id(), w = tid / kWave;
  const int64_t n_vis = visible(a, r);
  if (c >= chunks_of(n_vis, a.CH)) return;
  if ((int64_t)a.k >= n_vis) return;

  find_bucket(a.ghist + (size_t)r * kBuckets, (uint32_t)a.k, tmp, sel);
  const uint32_t T1 = sel[0];
  if (c == 0 && tid == 0) {
    a.rowsel[4 * r] = sel[0];
    a.rowsel[4 * r + 1] = sel[1];
  }

  const uint32_t* keys_row = a.keys + (size_t)r * a.n_cap;
  uint64_t* cand_chunk = a.cand + (size_t)r * a.n_cap + (size_t)c * a.CH;
  const int64_t j0 = (int64_t)c * a.CH;
  uint32_t gt = 0, ncand = 0;
  for (int it = 0; it < a.CH / kNT; ++it) {
    const int64_t jb = j0 + (int64_t)it * kNT;
    if (jb >= n_vis) break;
    const int64_t j = jb + tid;
    const bool valid = j < n_vis;
    const uint32_t key = valid ? keys_row[j] : 0u;
    const uint32_t bk = key >> kBucketShift;
    gt += (valid && bk > T1) ? 1u : 0u;
    const bool isc = valid && bk == T1;
    uint32_t tot;
    const uint32_t slot = block_rank(isc, wcnt, &tot);
    if (isc) {
      cand_chunk[ncand + slot] = composite(key, (uint32_t)j);
      atomicAdd(&a.ghist2[(size_t)r * kBuckets + ((key >> 10) & 2047u)], 1u);
    }
    ncand += tot;
  }
  const uint32_t gtt = wave_sum_u32(gt);
  if (lane == 0) tmp[w] = gtt;
  __syncthreads();
  if (tid == 0) {
    uint32_t t = 0;
    for (int i = 0; i < kNT / kWave; ++i) t += tmp[i];
    a.cgt[(size_t)r * a.C + c] = t;
    a.ccnt[(size_t)r * a.C + c] = ncand;
  }
}

// ------------------------------------------------------------------ select
// Index of the bin holding the rank-th largest element of a descending
// histogram h[0..NB) (bin NB-1 holds the largest values); rank is 1-based.
// Returns the bin and the rank left inside it.  Every thread must call.
template <int NB>
CLSA_DEV void find_bin_desc(const uint32_t* h, uint32_t rank, uint32_t* tmp, uint32_t* out2) {
  constexpr int PER = NB / kNT;
  const int tid = threadIdx.x;
  uint32_t v[PER], sum = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    v[i] = h[NB - 1 - PER * tid - i];
    sum += v[i];
  }
  const uint32_t incl = block_incl_scan<kNT>(sum, tmp);
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

// rank-th largest (1-based) of distinct 42-bit composites, visited through
// `visit(f)`, which calls f(v) once per element, split over threads.  Slow
// path for degenerate inputs only.
template <class Visit>
CLSA_DEV uint64_t block_select_desc(Visit visit, uint32_t rank, uint32_t* h256, uint32_t* tmp,
                                    uint32_t* bcast) {
  const int tid = threadIdx.x;
  uint64_t prefix = 0, pmask = 0;
  for (int shift = 40; shift >= 0; shift -= 8) {
    h256[tid] = 0u;
    __syncthreads();
    visit([&](uint64_t v) {
      if ((v & pmask) == prefix) atomicAdd(&h256[(uint32_t)(v >> shift) & 255u], 1u);
    });
    __syncthreads();
    find_bin_desc<256>(h256, rank, tmp, bcast);
    prefix |= (uint64_t)bcast[0] << shift;
    pmask |= (uint64_t)0xFFu << shift;
    rank = bcast[1];
    __syncthreads();
  }
  return prefix;
}

constexpr int kSmall = 256;  // boundary-bin candidates ranked pairwise

__global__ __launch_bounds__(kNT) void route_select(RouteArgs a) {
  __shared__ uint64_t small[kSmall];
  __shared__ uint32_t csel[kMaxChunks];
  __shared__ uint32_t h256[256];
  __shared__ uint32_t tmp[kNT / kWave];
  __shared__ uint32_t bc[4];
  __shared__ uint32_t nsmall;

  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t n_vis = visible(a, r);
  if ((int64_t)a.k >= n_vis) return;
  const int64_t nch = chunks_of(n_vis, a.CH);
  const uint32_t r1 = a.rowsel[4 * r + 1];
  const uint32_t* ccnt_row = a.ccnt + (size_t)r * a.C;
  const uint32_t* cgt_row = a.cgt + (size_t)r * a.C;
  const uint64_t* cand_row = a.cand + (size_t)r * a.n_cap;

  // second-level bin T2 of the r1-th largest candidate, and the rank left in it
  if (tid == 0) nsmall = 0;
  find_bin_desc<kBuckets>(a.ghist2 + (size_t)r * kBuckets, r1, tmp, bc);
  const uint32_t T2 = bc[0];
  const uint32_t r2 = bc[1];
  __syncthreads();

  // each thread owns whole chunks: count candidates above T2, collect those in T2
  const int per = (int)ceil_div64(nch, kNT);
  const int64_t cs = (int64_t)tid * per;
  for (int i = 0; i < per; ++i) {
    const int64_t c = cs + i;
    if (c >= nch) break;
    const uint32_t nc = ccnt_row[c];
    const uint64_t* cp = cand_row + c * a.CH;
    uint32_t above = 0;
#pragma unroll 8
    for (uint32_t e = 0; e < nc; ++e) {
      const uint64_t v = cp[e];
      const uint32_t b2 = (uint32_t)(v >> 42) & 2047u;
      above += b2 > T2 ? 1u : 0u;
      if (b2 == T2) {
        const uint32_t slot = atomicAdd(&nsmall, 1u);
        if (slot < (uint32_t)kSmall) small[slot] = v;
      }
    }
    csel[c] = above;
  }
  __syncthreads();
  const uint32_t m = nsmall;
  if (m <= (uint32_t)kSmall) {
    // the r2-th largest of m distinct composites: count the larger ones
    if (tid < (int)m) {
      const uint64_t v = small[tid];
      uint32_t larger = 0;
      for (uint32_t j = 0; j < m; ++j) larger += small[j] > v ? 1u : 0u;
      if (larger + 1 == r2) {
        bc[2] = (uint32_t)v;
        bc[3] = (uint32_t)(v >> 32);
      }
    }
  } else {
    // degenerate: too many equal top bits; radix select over the low 42 bits
    auto visit = [&](auto f) {
      for (int i = 0; i < per; ++i) {
        const int64_t c = cs + i;
        if (c >= nch) break;
        const uint32_t nc = ccnt_row[c];
        for (uint32_t e = 0; e < nc; ++e) {
          const uint64_t v = cand_row[c * a.CH + e];
          if (((uint32_t)(v >> 42) & 2047u) == T2) f(v & ((1ull << 42) - 1));
        }
      }
    };
    const uint64_t low = block_select_desc(visit, r2, h256, tmp, bc);
    if (tid == 0) {
      const uint64_t v = low | ((uint64_t)T2 << 42);
      bc[2] = (uint32_t)v;
      bc[3] = (uint32_t)(v >> 32);
    }
  }
  __syncthreads();
  const uint64_t Tc = ((uint64_t)bc[3] << 32) | bc[2];

  // selected boundary-bin candidates, per chunk
  if (m <= (uint32_t)kSmall) {
    for (uint32_t i = tid; i < m; i += kNT)
      if (small[i] >= Tc) atomicAdd(&csel[(~(uint32_t)small[i]) / (uint32_t)a.CH], 1u);
  } else {
    for (int i = 0; i < per; ++i) {
      const int64_t c = cs + i;
      if (c >= nch) break;
      const uint32_t nc = ccnt_row[c];
      uint32_t add = 0;
      for (uint32_t e = 0; e < nc; ++e) {
        const uint64_t v = cand_row[c * a.CH + e];
        add += (((uint32_t)(v >> 42) & 2047u) == T2 && v >= Tc) ? 1u : 0u;
      }
      csel[c] += add;
    }
  }
  __syncthreads();

  // output offset of every chunk: keys above T1 plus selected candidates
  uint32_t loc = 0;
  for (int i = 0; i < per; ++i)
    if (cs + i < nch) loc += cgt_row[cs + i] + csel[cs + i];
  const uint32_t incl = block_incl_scan<kNT>(loc, tmp);
  uint32_t run = incl - loc;
  uint32_t* off_row = a.off + (size_t)r * a.C;
  for (int i = 0; i < per; ++i) {
    if (cs + i < nch) {
      off_row[cs + i] = run;
      run += cgt_row[cs + i] + csel[cs + i];
    }
  }
  if (tid == 0) {
    a.rowsel[4 * r + 2] = (uint32_t)Tc;
    a.rowsel[4 * r + 3] = (uint32_t)(Tc >> 32);
  }
}

// ----------------------------------------------------------------- compact
template <bool TOPK>
__global__ __launch_bounds__(kNT) void route_compact(RouteArgs a) {
  __shared__ uint32_t tmp[kNT / kWave];
  __shared__ uint32_t wcnt[kNT / kWave];

  const int c = blockIdx.x, r = blockIdx.y;
  const int tid = threadIdx.x;
  const int64_t n_vis = visible(a, r);
  const int64_t nch = chunks_of(n_vis, a.CH);
  if (c >= nch) return;
  const uint32_t* keys_row = a.keys + (size_t)r * a.n_cap;
  int32_t* out = a.idx + (size_t)r * a.cap;
  const int64_t j0 = (int64_t)c * a.CH;
  const uint32_t* cgt_row = a.cgt + (size_t)r * a.C;

  // mode: 0 all visible keys, 1 top-k rule, 2 threshold rule
  int mode = 2;
  uint32_t count = 0, T1 = 0, thr = 0;
  uint64_t Tc = 0;
  int64_t run = 0;
  if (TOPK) {
    if ((int64_t)a.k >= n_vis) {
      mode = 0;
      count = (uint32_t)n_vis;
      run = j0;
    } else {
      mode = 1;
      count = (uint32_t)a.k;
      T1 = a.rowsel[4 * r];
      Tc = ((uint64_t)a.rowsel[4 * r + 3] << 32) | a.rowsel[4 * r + 2];
      run = a.off[(size_t)r * a.C + c];
    }
  } else {
    thr = score_key(a.tau[r]);
    count = block_sum_prefix(cgt_row, nch, tmp);  // true set size
    run = block_sum_prefix(cgt_row, c, tmp);
  }

  for (int it = 0; it < a.CH / kNT; ++it) {
    const int64_t jb = j0 + (int64_t)it * kNT;
    if (jb >= n_vis) break;
    const int64_t j = jb + tid;
    bool p = j < n_vis;
    if (p && mode != 0) {
      const uint32_t key = keys_row[j];
      if (mode == 2) {
        p = key >= thr;
      } else {
        const uint32_t bk = key >> kBucketShift;
        p = bk > T1 || (bk == T1 && composite(key, (uint32_t)j) >= Tc);
      }
    }
    uint32_t tot;
    const uint32_t slot = block_rank(p, wcnt, &tot);
    if (p) {
      const int64_t o = run + slot;
      if (o < a.cap) out[o] = (int32_t)j;
    }
    run += tot;
  }

  if (c == 0) {
    if (tid == 0) a.counts[r] = (int32_t)count;
    const int64_t first = count < (uint32_t)a.cap ? (int64_t)count : (int64_t)a.cap;
    for (int64_t i = first + tid; i < a.cap; i += kNT) out[i] = -1;
  }
}

// ------------------------------------------------------------------- host
struct Layout {
  int CH, C;
  size_t o_gh, o_gh2, ctrl_end, o_rowsel, o_cgt, o_ccnt, o_off, o_keys, o_cand, total;
};

Layout make_layout(int64_t R, int64_t n_cap, bool topk) {
  Layout L{};
  int64_t CH = 1024;
  if (ceil_div64(n_cap, CH) > kMaxChunks) CH = (ceil_div64(n_cap, kMaxChunks) + 255) / 256 * 256;
  L.CH = (int)CH;
  L.C = (int)ceil_div64(n_cap, CH);
  size_t o = 0;
  L.o_gh = o;
  o = align_up(o + (topk ? (size_t)R * kBuckets * 4 : 0), 256);
  L.o_gh2 = o;
  o = align_up(o + (topk ? (size_t)R * kBuckets * 4 : 0), 256);
  L.ctrl_end = o;
  L.o_rowsel = o; o = align_up(o + (size_t)R * 16, 256);
  L.o_cgt = o; o = align_up(o + (size_t)R * L.C * 4, 256);
  L.o_ccnt = o; o = align_up(o + (topk ? (size_t)R * L.C * 4 : 0), 256);
  L.o_off = o; o = align_up(o + (topk ? (size_t)R * L.C * 4 : 0), 256);
  L.o_keys = o; o = align_up(o + (size_t)R * n_cap * 4, 256);
  L.o_cand = o; o = align_up(o + (topk ? (size_t)R * n_cap * 8 : 0), 256);
  L.total = o;
  return L;
}

bool shape_ok(int B, int M, int d, int64_t n_cap, int cap) {
  if (B < 1 || M < 1 || cap < 1) return false;
  if (d != 32 && d != 64 && d != 128) return false;
  if (n_cap < 1 || n_cap > (int64_t)0x7fffffff) return false;
  const int64_t R = (int64_t)B * M;
  if (R > 65535) return false;  // rows map to gridDim.y
  return true;
}

template <int MODE>
void launch_score(const RouteArgs& a, clsa_dtype dt, int d, dim3 grid, hipStream_t s) {
  if (dt == CLSA_BF16) {
    if (d == 32) hipLaunchKernelGGL((route_score<uint16_t, 32, MODE>), grid, dim3(kNT), 0, s, a);
    if (d == 64) hipLaunchKernelGGL((route_score<uint16_t, 64, MODE>), grid, dim3(kNT), 0, s, a);
    if (d == 128) hipLaunchKernelGGL((route_score<uint16_t, 128, MODE>), grid, dim3(kNT), 0, s, a);
  } else if constexpr (MODE != kFilter) {
    if (d == 32) hipLaunchKernelGGL((route_score<float, 32, MODE>), grid, dim3(kNT), 0, s, a);
    if (d == 64) hipLaunchKernelGGL((route_score<float, 64, MODE>), grid, dim3(kNT), 0, s, a);
    if (d == 128) hipLaunchKernelGGL((route_score<float, 128, MODE>), grid, dim3(kNT), 0, s, a);
  }
}

// Filter path workspace: keys per chunk chosen so that the score pass has
// at least about a thousand workgroups (256 .. 2048 keys, a multiple of the
// block; 8 rows at 128K take 1024-key chunks, 32 rows 2048); per row the
// samples, a candidate count per chunk and C x segcap candidate entries.
// segcap gives a row at least 8192 entries (the select takes at most 6144)
// and every chunk at least 32: a full row at 128K expects about 28 per
// 1024-key chunk against a share of 64; shorter rows share the same
// entries among fewer chunks.
struct FilterLayout {
  int CH, C, segcap;
  size_t o_samp, o_cnt, o_cand, total;
};

FilterLayout filter_layout(int64_t R, int64_t n_cap) {
  FilterLayout L{};
  int64_t CH = kMaxFilterCH;
  while (CH > kNT && R * ceil_div64(n_cap, CH) < 1024) CH /= 2;
  L.CH = (int)CH;
  L.C = (int)ceil_div64(n_cap, CH);
  int64_t sc = ceil_div64(8192, L.C);
  if (sc < 32) sc = 32;
  L.segcap = (int)(sc < CH ? sc : CH);
  size_t o = 0;
  L.o_samp = o; o = align_up(o + (size_t)R * kRowSamples * 2, 256);
  L.o_cnt = o; o = align_up(o + (size_t)R * L.C * 4, 256);
  L.o_cand = o; o = align_up(o + (size_t)R * L.C * L.segcap * 8, 256);
  L.total = o;
  return L;
}

RouteArgs fill_args(const Layout& L, void* ws, const void* q_idx, const void* K_idx, int B, int M,
                    int64_t n_cap, const int32_t* n_ctx, int64_t q_pos0, int k,
                    const float* tau, int32_t* idx, int32_t* counts, int cap) {
  char* base = static_cast<char*>(ws);
  RouteArgs a{};
  a.q = q_idx;
  a.K = K_idx;
  a.n_ctx = n_ctx;
  a.tau = tau;
  a.idx = idx;
  a.counts = counts;
  a.n_cap = n_cap;
  a.q_pos0 = q_pos0 < 0 ? -1 : q_pos0;
  a.B = B;
  a.M = M;
  a.k = k;
  a.cap = cap;
  a.CH = L.CH;
  a.C = L.C;
  a.ghist = reinterpret_cast<uint32_t*>(base + L.o_gh);
  a.ghist2 = reinterpret_cast<uint32_t*>(base + L.o_gh2);
  a.rowsel = reinterpret_cast<uint32_t*>(base + L.o_rowsel);
  a.cgt = reinterpret_cast<uint32_t*>(base + L.o_cgt);
  a.ccnt = reinterpret_cast<uint32_t*>(base + L.o_ccnt);
  a.off = reinterpret_cast<uint32_t*>(base + L.o_off);
  a.keys = reinterpret_cast<uint32_t*>(base + L.o_keys);
  a.cand = reinterpret_cast<uint64_t*>(base + L.o_cand);
  return a;
}

}  // namespace

// Block routing on the matrix cores (clsa_prefill.hip): bf16 keys, many
// query rows per sequence.
bool block_route_applies(int M, int d, int64_t n_cap, int k, clsa_dtype dt);
size_t block_route_workspace(int B, int M, int d, int64_t n_cap);
int block_route(const void* q_idx, const void* K_idx, int B, int M, int d, int64_t n_cap,
                const int32_t* n_ctx, int64_t q_pos0, int k, int32_t* idx, int32_t* counts,
                int cap, void* ws, hipStream_t s);
// Threshold and select of the filter path (clsa_prefill.hip).
bool seg_route_applies(int M, int d, int64_t n_cap, int k, clsa_dtype dt);
void seg_route_sample(const void* q_idx, const void* K_idx, int B, int M, int d, int64_t n_cap,
                      const int32_t* n_ctx, int64_t q_pos0, int k, uint16_t* samp, hipStream_t s);
void seg_route_select(const void* q_idx, const void* K_idx, int B, int M, int d, int64_t n_cap,
                      const int32_t* n_ctx, int64_t q_pos0, int k, int32_t* idx, int32_t* counts,
                      int cap, int chunk_keys, int nchunks, int segcap, uint32_t* segcnt,
                      uint64_t* seg, hipStream_t s);
}  // namespace clsa

using namespace clsa;

extern "C" size_t clsa_route_workspace_size(int B, int M, int d, int64_t n_cap, int k, int cap,
                                            clsa_dtype dt) {
  if (!shape_ok(B, M, d, n_cap, cap) || k < 1) return 0;
  if (block_route_applies(M, d, n_cap, k, dt)) return block_route_workspace(B, M, d, n_cap);
  if (seg_route_applies(M, d, n_cap, k, dt)) return filter_layout((int64_t)B * M, n_cap).total;
  return make_layout((int64_t)B * M, n_cap, true).total;
}

namespace clsa {
namespace {
// Argument checks of clsa_route that need no workspace: the status to
// return, CLSA_OK when the call may proceed.
int route_args_status(const void* q_idx, const void* K_idx, int B, int M, int d, int64_t n_cap,
                      int k, clsa_dtype dt, const int32_t* idx, const int32_t* counts, int cap) {
  if (dt != CLSA_F32 && dt != CLSA_BF16) return CLSA_ERR_UNSUPPORTED_DTYPE;
  if (!q_idx || !K_idx || !idx || !counts) return CLSA_ERR_INVALID;
  if (!shape_ok(B, M, d, n_cap, cap) || k < 1 || cap < k) return CLSA_ERR_INVALID;
  return CLSA_OK;
}

// clsa_route on a workspace `ws` of `ws_bytes`: picks the block, filter or
// exhaustive path and enqueues its kernels.  Every path clears what it
// needs zeroed with kernels, so the workspace may hold anything on entry.
int route_call(const void* q_idx, const void* K_idx, int B, int M, int d, int64_t n_cap,
               const int32_t* n_ctx, int64_t q_pos0, int k, clsa_dtype dt, int32_t* idx,
               int32_t* counts, int cap, void* ws, size_t ws_bytes, hipStream_t s) {
  const int st = route_args_status(q_idx, K_idx, B, M, d, n_cap, k, dt, idx, counts, cap);
  if (st != CLSA_OK) return st;
  if (block_route_applies(M, d, n_cap, k, dt)) {
    if (!ws || ws_bytes < block_route_workspace(B, M, d, n_cap)) return CLSA_ERR_WORKSPACE;
    return block_route(q_idx, K_idx, B, M, d, n_cap, n_ctx, q_pos0, k, idx, counts, cap, ws, s);
  }
  const int64_t R = (int64_t)B * M;
  if (seg_route_applies(M, d, n_cap, k, dt)) {
    const FilterLayout F = filter_layout(R, n_cap);
    if (!ws || ws_bytes < F.total) return CLSA_ERR_WORKSPACE;
    char* base = static_cast<char*>(ws);
    RouteArgs a{};
    a.q = q_idx;
    a.K = K_idx;
    a.n_ctx = n_ctx;
    a.n_cap = n_cap;
    a.q_pos0 = q_pos0 < 0 ? -1 : q_pos0;
    a.B = B;
    a.M = M;
    a.k = k;
    a.cap = cap;
    a.CH = F.CH;
    a.C = F.C;
    a.samp = reinterpret_cast<const uint16_t*>(base + F.o_samp);
    a.segcnt = reinterpret_cast<uint32_t*>(base + F.o_cnt);
    a.seg = reinterpret_cast<uint64_t*>(base + F.o_cand);
    a.segcap = F.segcap;
    seg_route_sample(q_idx, K_idx, B, M, d, n_cap, n_ctx, q_pos0, k,
                     reinterpret_cast<uint16_t*>(base + F.o_samp), s);
    launch_score<kFilter>(a, dt, d, dim3((unsigned)F.C, (unsigned)R), s);
    seg_route_select(q_idx, K_idx, B, M, d, n_cap, n_ctx, q_pos0, k, idx, counts, cap, F.CH, F.C,
                     F.segcap, a.segcnt, a.seg, s);
    return hipGetLastError() == hipSuccess ? CLSA_OK : CLSA_ERR_HIP;
  }
  const Layout L = make_layout(R, n_cap, true);
  if (!ws || ws_bytes < L.total) return CLSA_ERR_WORKSPACE;
  const RouteArgs a = fill_args(L, ws, q_idx, K_idx, B, M, n_cap, n_ctx, q_pos0, k, nullptr,
                                idx, counts, cap);
  if (zero_fill(ws, L.ctrl_end, s) != hipSuccess) return CLSA_ERR_HIP;
  const dim3 grid((unsigned)L.C, (unsigned)R);
  launch_score<kHist>(a, dt, d, grid, s);
  hipLaunchKernelGGL(route_cands, grid, dim3(kNT), 0, s, a);
  hipLaunchKernelGGL(route_select, dim3((unsigned)R), dim3(kNT), 0, s, a);
  hipLaunchKernelGGL(route_compact<true>, grid, dim3(kNT), 0, s, a);
  return hipGetLastError() == hipSuccess ? CLSA_OK : CLSA_ERR_HIP;
}
}  // namespace
}  // namespace clsa

extern "C" int clsa_route(const void* q_idx, const void* K_idx, int B, int M, int d,
                          int64_t n_cap, const int32_t* n_ctx, int64_t q_pos0, int k,
                          clsa_dtype dt, int32_t* idx, int32_t* counts, int cap, void* ws,
                          size_t ws_bytes, void* stream) {
  return route_call(q_idx, K_idx, B, M, d, n_cap, n_ctx, q_pos0, k, dt, idx, counts, cap, ws,
                    ws_bytes, static_cast<hipStream_t>(stream));
}

// ------------------------------------------------------- no-allocation routing
// clsa_route_static runs clsa_route's kernels on a fixed device array in
// place of a caller workspace.  `scratch` is a host-side stand-in for that
// array; host code only ever uses the address hipGetSymbolAddress returns
// for it on the current device (each GPU holds its own copy).
static __device__ __align__(256) unsigned char scratch[CLSA_STATIC_SCRATCH_BYTES];

namespace clsa {
namespace {
constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// Device address of `scratch` on the calling thread's current device,
// looked up once per device and kept.
int static_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return CLSA_ERR_HIP;
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = p;
  });
  if (g_scratch_err[dev] != hipSuccess || g_scratch_ptr[dev] == nullptr) return CLSA_ERR_HIP;
  *out = g_scratch_ptr[dev];
  return CLSA_OK;
}
}  // namespace
}  // namespace clsa

extern "C" int clsa_route_static(const void* q_idx, const void* K_idx, int B, int M, int d,
                                 int64_t n_cap, const int32_t* n_ctx, int64_t q_pos0, int k,
                                 clsa_dtype dt, int32_t* idx, int32_t* counts, int cap,
                                 void* stream) {
  const int st = route_args_status(q_idx, K_idx, B, M, d, n_cap, k, dt, idx, counts, cap);
  if (st != CLSA_OK) return st;
  if (clsa_route_workspace_size(B, M, d, n_cap, k, cap, dt) > (size_t)CLSA_STATIC_SCRATCH_BYTES)
    return CLSA_ERR_SCRATCH_LIMIT;
  void* ptr = nullptr;
  const int sst = static_scratch(&ptr);
  if (sst != CLSA_OK) return sst;
  return route_call(q_idx, K_idx, B, M, d, n_cap, n_ctx, q_pos0, k, dt, idx, counts, cap, ptr,
                    (size_t)CLSA_STATIC_SCRATCH_BYTES, static_cast<hipStream_t>(stream));
}

extern "C" size_t clsa_route_threshold_workspace_size(int B, int M, int d, int64_t n_cap, int cap,
                                                      clsa_dtype dt) {
  (void)dt;
  if (!shape_ok(B, M, d, n_cap, cap)) return 0;
  return make_layout((int64_t)B * M, n_cap, false).total;
}

extern "C" int clsa_route_threshold(const void* q_idx, const void* K_idx, int B, int M, int d,
                                    int64_t n_cap, const int32_t* n_ctx, int64_t q_pos0,
                                    const float* tau, clsa_dtype dt, int32_t* idx,
                                    int32_t* counts, int cap, void* ws, size_t ws_bytes,
                                    void* stream) {
  if (dt != CLSA_F32 && dt != CLSA_BF16) return CLSA_ERR_UNSUPPORTED_DTYPE;
  if (!q_idx || !K_idx || !tau || !idx || !counts) return CLSA_ERR_INVALID;
  if (!shape_ok(B, M, d, n_cap, cap)) return CLSA_ERR_INVALID;
  const int64_t R = (int64_t)B * M;
  const Layout L = make_layout(R, n_cap, false);
  if (!ws || ws_bytes < L.total) return CLSA_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const RouteArgs a = fill_args(L, ws, q_idx, K_idx, B, M, n_cap, n_ctx, q_pos0, 1, tau, idx,
                                counts, cap);
  const dim3 grid((unsigned)L.C, (unsigned)R);
  launch_score<kCount>(a, dt, d, grid, s);
  hipLaunchKernelGGL(route_compact<false>, grid, dim3(kNT), 0, s, a);
  return hipGetLastError() == hipSuccess ? CLSA_OK : CLSA_ERR_HIP;
}

// ------------------------------------------------- cross-layer aggregation
// clsa_route_aggregated: the exhaustive path with H index heads whose scores
// are summed per key (see clsa.h).
extern "C" size_t clsa_route_aggregated_workspace_size(int H, int B, int M, int d, int64_t n_cap,
                                                       int k, int cap, clsa_dtype dt) {
  (void)dt;
  if (H < 1 || H > kMaxHeads || !shape_ok(B, M, d, n_cap, cap) || k < 1) return 0;
  return make_layout((int64_t)B * M, n_cap, true).total;
}

extern "C" int clsa_route_aggregated(int H, const void* const* q_idx, const void* const* K_idx,
                                     int B, int M, int d, int64_t n_cap, const int32_t* n_ctx,
                                     int64_t q_pos0, int k, clsa_dtype dt, int32_t* idx,
                                     int32_t* counts, int cap, void* ws, size_t ws_bytes,
                                     void* stream) {
  if (dt != CLSA_F32 && dt != CLSA_BF16) return CLSA_ERR_UNSUPPORTED_DTYPE;
  if (H < 1 || H > kMaxHeads || !q_idx || !K_idx || !idx || !counts) return CLSA_ERR_INVALID;
  for (int h = 0; h < H; ++h)
    if (!q_idx[h] || !K_idx[h]) return CLSA_ERR_INVALID;
  if (!shape_ok(B, M, d, n_cap, cap) || k < 1 || cap < k) return CLSA_ERR_INVALID;
  const int64_t R = (int64_t)B * M;
  const Layout L = make_layout(R, n_cap, true);
  if (!ws || ws_bytes < L.total) return CLSA_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  RouteArgs a = fill_args(L, ws, q_idx[0], K_idx[0], B, M, n_cap, n_ctx, q_pos0, k, nullptr, idx,
                          counts, cap);
  a.H = H;
  for (int h = 0; h < H; ++h) {
    a.qh[h] = q_idx[h];
    a.Kh[h] = K_idx[h];
  }
  if (zero_fill(ws, L.ctrl_end, s) != hipSuccess) return CLSA_ERR_HIP;
  const dim3 grid((unsigned)L.C, (unsigned)R);
  launch_score<kHist>(a, dt, d, grid, s);
  hipLaunchKernelGGL(route_cands, grid, dim3(kNT), 0, s, a);
  hipLaunchKernelGGL(route_select, dim3((unsigned)R), dim3(kNT), 0, s, a);
  hipLaunchKernelGGL(route_compact<true>, grid, dim3(kNT), 0, s, a);
  return hipGetLastError() == hipSuccess ? CLSA_OK : CLSA_ERR_HIP;
}

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
// Kernels (grid = chunks x rows; a chunk is CH consecutive keys of a row):
//   route_score    s_j = q . K_idx[j] (fp32 accumulation, coalesced 16-byte
//                  loads + a butterfly reduce-scatter across the lanes of a
//                  key row), stores order-preserving uint32 keys, and either
//                  builds the row's 2048-bucket histogram of the top 11 key
//                  bits (top-k) or counts keys >= key(tau) per chunk
//                  (threshold).  The last workgroup of a row finishes the
//                  row: it finds the bucket holding the k-th largest key, or
//                  scans the per-chunk counts into output offsets.
//   route_cands    (top-k) collects the keys of that bucket as candidates
//                  (composite key: low 21 key bits, then inverted position so
//                  lower positions win ties) and counts keys above it per
//                  chunk; the last workgroup runs an exact LDS radix select
//                  over the candidates and scans per-chunk output offsets.
//   route_compact  writes selected positions in ascending order with wave
//                  ballots and per-chunk offsets, pads with -1, sets counts.
// Completion of a row is detected with a per-row arrival counter (release /
// acquire at agent scope); no workgroup ever waits on another.
#include "clsa_common.h"

namespace clsa {
namespace {

constexpr int kNT = 256;             // threads per workgroup
constexpr int kBuckets = 2048;       // histogram of the top 11 key bits
constexpr int kBucketShift = 21;
constexpr uint32_t kLowMask = (1u << kBucketShift) - 1u;
constexpr int kMaxChunks = 4096;     // chunks per row (LDS table in route_cands)
constexpr int kCandLds = 6144;       // candidates kept in LDS for the select

enum : uint32_t { kModeTopk = 0, kModeAll = 1, kModeThresh = 2 };

struct RowInfo {
  uint32_t mode;
  uint32_t n_vis;
  uint32_t count;  // keys to emit (top-k) or true set size (threshold)
  uint32_t T1;     // top-k: bucket of the count-th key; threshold: key(tau)
  uint32_t r1;     // top-k: keys to take from bucket T1
  uint32_t pad;
  uint64_t Tc;     // top-k: composite key of the last taken candidate
};

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
  uint32_t* ticket1;      // [R]
  uint32_t* ticket2;      // [R]
  uint32_t* ccount;       // [R]
  uint32_t* ghist;        // [R][2048]
  RowInfo* info;          // [R]
  uint32_t* cnt;          // [R][C] keys above T1 (top-k) / keys >= tau (threshold)
  uint32_t* coff;         // [R][C] output offset of each chunk
  uint32_t* keys;         // [R][n_cap]
  uint64_t* cand;         // [R][n_cap]
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
  CLSA_DEV static float dot(const uint4 v, const float* qf) {
    float s = qf[0] * __uint_as_float(v.x);
    s = fmaf(qf[1], __uint_as_float(v.y), s);
    s = fmaf(qf[2], __uint_as_float(v.z), s);
    s = fmaf(qf[3], __uint_as_float(v.w), s);
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
  CLSA_DEV static float dot(const uint4 v, const float* qf) {
    // bf16 x bf16 products are exact in fp32, so fma and mul+add agree.
    float s = qf[0] * bf16_lo(v.x);
    s = fmaf(qf[1], bf16_hi(v.x), s);
    s = fmaf(qf[2], bf16_lo(v.y), s);
    s = fmaf(qf[3], bf16_hi(v.y), s);
    s = fmaf(qf[4], bf16_lo(v.z), s);
    s = fmaf(qf[5], bf16_hi(v.z), s);
    s = fmaf(qf[6], bf16_lo(v.w), s);
    s = fmaf(qf[7], bf16_hi(v.w), s);
    return s;
  }
  CLSA_DEV static void load_q(const void* q, size_t off, float* qf) {
    const uint16_t* p = static_cast<const uint16_t*>(q) + off;
#pragma unroll
    for (int e = 0; e < 8; ++e) qf[e] = __uint_as_float((uint32_t)p[e] << 16);
  }
};

// U partial sums per lane, U consecutive lanes per key row.  After the
// butterfly, lane with in-group position p holds the full sum of partial
// index p.  The addition tree is the same for every partial index, so
// identical key rows give bit-identical scores.
template <int U>
CLSA_DEV float reduce_scatter(float (&v)[U], int lane) {
#pragma unroll
  for (int m = U / 2; m >= 1; m >>= 1) {
    const bool up = (lane & m) != 0;
#pragma unroll
    for (int i = 0; i < m; ++i) {
      const float send = up ? v[i] : v[i + m];
      const float keep = up ? v[i + m] : v[i];
      v[i] = keep + __shfl_xor(send, m);
    }
  }
  return v[0];
}

// ------------------------------------------------------------------- score
template <typename T, int D, uint32_t MODE>
__global__ __launch_bounds__(kNT) void route_score(RouteArgs a) {
  constexpr int kEPL = Elem<T>::kPer16;        // elements per 16-byte segment
  constexpr int kLPR = D / kEPL;               // lanes per key row
  constexpr int kKPI = kWave / kLPR;           // key rows per wave load
  constexpr int kU = kLPR;                     // loads per lane per wave pass
  static_assert(kLPR >= 2 && kLPR <= 32, "unsupported row width");

  __shared__ uint32_t hist[kBuckets];
  __shared__ uint32_t scan_tmp[kNT / kWave];
  __shared__ uint32_t s_last;

  const int c = blockIdx.x, r = blockIdx.y;
  const int tid = threadIdx.x, lane = lane_id(), w = tid / kWave;
  const int b = r / a.M;
  const int64_t n_vis = visible(a, r);
  const int64_t nch = chunks_of(n_vis, a.CH);
  if (c >= nch) return;

  if (MODE == kModeTopk) {
    const int64_t k_eff = a.k < n_vis ? a.k : n_vis;
    if (k_eff >= n_vis) {  // every visible key is selected: no scoring needed
      if (c == 0 && tid == 0) {
        RowInfo ri{};
        ri.mode = kModeAll;
        ri.n_vis = (uint32_t)n_vis;
        ri.count = (uint32_t)n_vis;
        a.info[r] = ri;
      }
      return;
    }
    for (int i = tid; i < kBuckets; i += kNT) hist[i] = 0u;
    __syncthreads();
  }
  uint32_t tkey = 0;
  if (MODE == kModeThresh) tkey = score_key(a.tau[r]);

  const int grp = lane / kLPR, pos = lane % kLPR;
  float qf[kEPL];
  Elem<T>::load_q(a.q, (size_t)r * D + (size_t)pos * kEPL, qf);

  const char* Kb = static_cast<const char*>(a.K) + (size_t)b * a.n_cap * D * sizeof(T);
  uint32_t* keys_row = a.keys + (size_t)r * a.n_cap;
  const int64_t j0 = (int64_t)c * a.CH;
  uint32_t n_ge = 0;

  for (int it = 0; it < a.CH / kNT; ++it) {
    const int64_t wbase = j0 + (int64_t)it * kNT + w * kWave;
    if (wbase >= n_vis) break;
    float part[kU];
    uint4 v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t j = wbase + u * kKPI + grp;
      const int64_t jj = j < n_vis ? j : 0;
      v[u] = *reinterpret_cast<const uint4*>(Kb + (size_t)jj * D * sizeof(T) + pos * 16);
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) part[u] = Elem<T>::dot(v[u], qf);
    const float s = reduce_scatter<kU>(part, lane);
    const int64_t j = wbase + pos * kKPI + grp;
    if (j < n_vis) {
      const uint32_t key = score_key(s);
      keys_row[j] = key;
      if (MODE == kModeTopk) atomicAdd(&hist[key >> kBucketShift], 1u);
      if (MODE == kModeThresh) n_ge += (key >= tkey) ? 1u : 0u;
    }
  }

  if (MODE == kModeTopk) {
    __syncthreads();
    uint32_t* gh = a.ghist + (size_t)r * kBuckets;
    for (int i = tid; i < kBuckets; i += kNT) {
      const uint32_t h = hist[i];
      if (h) atomicAdd(&gh[i], h);
    }
  } else {
    const uint32_t tot = wave_sum_u32(n_ge);
    if (lane == 0) scan_tmp[w] = tot;
    __syncthreads();
    if (tid == 0) {
      uint32_t t = 0;
      for (int i = 0; i < kNT / kWave; ++i) t += scan_tmp[i];
      a.cnt[(size_t)r * a.C + c] = t;
    }
  }

  __syncthreads();
  if (tid == 0) s_last = (arrive_release(&a.ticket1[r]) == (uint32_t)(nch - 1)) ? 1u : 0u;
  __syncthreads();
  if (!s_last) return;
  acquire_device();

  if (MODE == kModeTopk) {
    // Find the bucket holding the k_eff-th largest key.  Thread t owns
    // buckets 2047-8t .. 2040-8t (descending).
    const uint32_t k_eff = (uint32_t)(a.k < n_vis ? a.k : n_vis);
    const uint32_t* gh = a.ghist + (size_t)r * kBuckets;
    uint32_t h[8], sum = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      h[i] = load_relaxed(&gh[kBuckets - 1 - 8 * tid - i]);
      sum += h[i];
    }
    const uint32_t incl = block_incl_scan<kNT>(sum, scan_tmp);
    const uint32_t excl = incl - sum;
    if (excl < k_eff && k_eff <= incl) {
      uint32_t acc = excl;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (acc + h[i] >= k_eff) {
          RowInfo ri{};
          ri.mode = kModeTopk;
          ri.n_vis = (uint32_t)n_vis;
          ri.count = k_eff;
          ri.T1 = (uint32_t)(kBuckets - 1 - 8 * tid - i);
          ri.r1 = k_eff - acc;
          a.info[r] = ri;
          break;
        }
        acc += h[i];
      }
    }
  } else {
    // Exclusive scan of the per-chunk counts -> output offsets.
    const int per = (int)ceil_div64(nch, kNT);
    const int64_t cs = (int64_t)tid * per;
    uint32_t loc = 0;
    for (int i = 0; i < per; ++i)
      if (cs + i < nch) loc += load_relaxed(&a.cnt[(size_t)r * a.C + cs + i]);
    const uint32_t incl = block_incl_scan<kNT>(loc, scan_tmp);
    uint32_t run = incl - loc;
    for (int i = 0; i < per; ++i) {
      if (cs + i < nch) {
        const uint32_t v = load_relaxed(&a.cnt[(size_t)r * a.C + cs + i]);
        a.coff[(size_t)r * a.C + cs + i] = run;
        run += v;
      }
    }
    if (tid == kNT - 1) {
      RowInfo ri{};
      ri.mode = kModeThresh;
      ri.n_vis = (uint32_t)n_vis;
      ri.count = incl;
      ri.T1 = tkey;
      a.info[r] = ri;
    }
  }
}

// ------------------------------------------------- exact radix select (LDS)
// rank-th largest (1-based) of n distinct 53-bit composites.  Values come
// from LDS when they fit, else from global memory.
CLSA_DEV uint64_t block_select_desc(const uint64_t* src, uint32_t n, uint32_t rank,
                                    uint32_t* h256, uint32_t* scan_tmp, uint32_t* bcast) {
  const int tid = threadIdx.x;
  uint64_t prefix = 0, pmask = 0;
  for (int shift = 48; shift >= 0; shift -= 8) {
    h256[tid] = 0u;
    __syncthreads();
    for (uint32_t i = tid; i < n; i += kNT) {
      const uint64_t v = src[i];
      if ((v & pmask) == prefix) atomicAdd(&h256[(uint32_t)(v >> shift) & 255u], 1u);
    }
    __syncthreads();
    const uint32_t cnt = h256[255 - tid];  // digits in descending order
    const uint32_t incl = block_incl_scan<kNT>(cnt, scan_tmp);
    const uint32_t excl = incl - cnt;
    if (excl < rank && rank <= incl) {
      bcast[0] = 255u - (uint32_t)tid;
      bcast[1] = rank - excl;
    }
    __syncthreads();
    prefix |= (uint64_t)bcast[0] << shift;
    pmask |= (uint64_t)0xFFu << shift;
    rank = bcast[1];
    __syncthreads();
  }
  return prefix;
}

// -------------------------------------------------------------- candidates
__global__ __launch_bounds__(kNT) void route_cands(RouteArgs a) {
  __shared__ uint64_t cbuf[kCandLds];
  __shared__ uint32_t csel[kMaxChunks];
  __shared__ uint32_t h256[256];
  __shared__ uint32_t scan_tmp[kNT / kWave];
  __shared__ uint32_t bcast[2];
  __shared__ uint32_t s_last;

  const int c = blockIdx.x, r = blockIdx.y;
  const int tid = threadIdx.x, lane = lane_id(), w = tid / kWave;
  const RowInfo ri = a.info[r];
  if (ri.mode != kModeTopk) return;
  const int64_t n_vis = ri.n_vis;
  const int64_t nch = chunks_of(n_vis, a.CH);
  if (c >= nch) return;

  const uint32_t* keys_row = a.keys + (size_t)r * a.n_cap;
  uint64_t* cand_row = a.cand + (size_t)r * a.n_cap;
  const int64_t j0 = (int64_t)c * a.CH;
  uint32_t gt = 0;
  for (int it = 0; it < a.CH / kNT; ++it) {
    const int64_t j = j0 + (int64_t)it * kNT + tid;
    const bool valid = j < n_vis;
    const uint32_t key = valid ? keys_row[j] : 0u;
    const uint32_t bk = key >> kBucketShift;
    gt += (valid && bk > ri.T1) ? 1u : 0u;
    const bool isc = valid && bk == ri.T1;
    const uint64_t mask = __ballot(isc);
    if (mask) {
      const int leader = __ffsll((unsigned long long)mask) - 1;
      uint32_t base = 0;
      if (lane == leader) base = atomicAdd(&a.ccount[r], (uint32_t)__popcll(mask));
      base = __shfl(base, leader);
      if (isc) cand_row[base + lanes_below(mask)] = composite(key, (uint32_t)j);
    }
  }
  const uint32_t tot = wave_sum_u32(gt);
  if (lane == 0) scan_tmp[w] = tot;
  __syncthreads();
  if (tid == 0) {
    uint32_t t = 0;
    for (int i = 0; i < kNT / kWave; ++i) t += scan_tmp[i];
    a.cnt[(size_t)r * a.C + c] = t;
  }
  __syncthreads();
  if (tid == 0) s_last = (arrive_release(&a.ticket2[r]) == (uint32_t)(nch - 1)) ? 1u : 0u;
  __syncthreads();
  if (!s_last) return;
  acquire_device();

  // ---- last workgroup of the row: exact select among the candidates ----
  const uint32_t n_c = load_relaxed(&a.ccount[r]);
  const uint64_t* src = cand_row;
  if (n_c <= (uint32_t)kCandLds) {
    for (uint32_t i = tid; i < n_c; i += kNT) cbuf[i] = cand_row[i];
    __syncthreads();
    src = cbuf;
  }
  const uint64_t Tc = block_select_desc(src, n_c, ri.r1, h256, scan_tmp, bcast);

  for (int64_t i = tid; i < nch; i += kNT) csel[i] = 0u;
  __syncthreads();
  for (uint32_t i = tid; i < n_c; i += kNT) {
    const uint64_t v = src[i];
    if (v >= Tc) {
      const uint32_t j = ~(uint32_t)v;
      atomicAdd(&csel[j / (uint32_t)a.CH], 1u);
    }
  }
  __syncthreads();
  const int per = (int)ceil_div64(nch, kNT);
  const int64_t cs = (int64_t)tid * per;
  uint32_t loc = 0;
  for (int i = 0; i < per; ++i)
    if (cs + i < nch) loc += load_relaxed(&a.cnt[(size_t)r * a.C + cs + i]) + csel[cs + i];
  const uint32_t incl = block_incl_scan<kNT>(loc, scan_tmp);
  uint32_t run = incl - loc;
  for (int i = 0; i < per; ++i) {
    if (cs + i < nch) {
      a.coff[(size_t)r * a.C + cs + i] = run;
      run += load_relaxed(&a.cnt[(size_t)r * a.C + cs + i]) + csel[cs + i];
    }
  }
  if (tid == 0) a.info[r].Tc = Tc;
}

// ----------------------------------------------------------------- compact
__global__ __launch_bounds__(kNT) void route_compact(RouteArgs a) {
  __shared__ uint32_t wcnt[kNT / kWave];
  const int c = blockIdx.x, r = blockIdx.y;
  const int tid = threadIdx.x, w = tid / kWave;
  const RowInfo ri = a.info[r];
  const int64_t n_vis = ri.n_vis;
  const int64_t nch = chunks_of(n_vis, a.CH);
  if (c >= nch) return;

  const uint32_t* keys_row = a.keys + (size_t)r * a.n_cap;
  int32_t* out = a.idx + (size_t)r * a.cap;
  const int64_t j0 = (int64_t)c * a.CH;
  int64_t run = (ri.mode == kModeAll) ? j0 : (int64_t)a.coff[(size_t)r * a.C + c];

  for (int it = 0; it < a.CH / kNT; ++it) {
    const int64_t jb = j0 + (int64_t)it * kNT;
    if (jb >= n_vis) break;
    const int64_t j = jb + tid;
    bool p = j < n_vis;
    if (p && ri.mode != kModeAll) {
      const uint32_t key = keys_row[j];
      if (ri.mode == kModeThresh) {
        p = key >= ri.T1;
      } else {
        const uint32_t bk = key >> kBucketShift;
        p = bk > ri.T1 || (bk == ri.T1 && composite(key, (uint32_t)j) >= ri.Tc);
      }
    }
    const uint64_t mask = __ballot(p);
    if (lane_id() == 0) wcnt[w] = (uint32_t)__popcll(mask);
    __syncthreads();
    uint32_t before = 0, total = 0;
#pragma unroll
    for (int i = 0; i < kNT / kWave; ++i) {
      before += (i < w) ? wcnt[i] : 0u;
      total += wcnt[i];
    }
    if (p) {
      const int64_t o = run + before + lanes_below(mask);
      if (o < a.cap) out[o] = (int32_t)j;
    }
    run += total;
    __syncthreads();
  }

  if (c == 0) {
    const uint32_t count = ri.count;
    if (tid == 0) a.counts[r] = (int32_t)count;
    const int64_t first = count < (uint32_t)a.cap ? (int64_t)count : (int64_t)a.cap;
    for (int64_t i = first + tid; i < a.cap; i += kNT) out[i] = -1;
  }
}

// ------------------------------------------------------------------- host
struct Layout {
  int CH, C;
  size_t o_t1, o_t2, o_cc, o_gh, ctrl_end, o_info, o_cnt, o_coff, o_keys, o_cand, total;
};

Layout make_layout(int64_t R, int64_t n_cap, bool topk) {
  Layout L{};
  int64_t CH = 1024;
  if (ceil_div64(n_cap, CH) > kMaxChunks) CH = (ceil_div64(n_cap, kMaxChunks) + 255) / 256 * 256;
  L.CH = (int)CH;
  L.C = (int)ceil_div64(n_cap, CH);
  size_t o = 0;
  L.o_t1 = o; o += (size_t)R * 4;
  L.o_t2 = o; o += topk ? (size_t)R * 4 : 0;
  L.o_cc = o; o += topk ? (size_t)R * 4 : 0;
  L.o_gh = o; o += topk ? (size_t)R * kBuckets * 4 : 0;
  o = align_up(o, 256);
  L.ctrl_end = o;
  L.o_info = o; o = align_up(o + (size_t)R * sizeof(RowInfo), 256);
  L.o_cnt = o; o = align_up(o + (size_t)R * L.C * 4, 256);
  L.o_coff = o; o = align_up(o + (size_t)R * L.C * 4, 256);
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

template <uint32_t MODE>
void launch_score(const RouteArgs& a, clsa_dtype dt, int d, dim3 grid, hipStream_t s) {
  if (dt == CLSA_BF16) {
    if (d == 32) hipLaunchKernelGGL((route_score<uint16_t, 32, MODE>), grid, dim3(kNT), 0, s, a);
    if (d == 64) hipLaunchKernelGGL((route_score<uint16_t, 64, MODE>), grid, dim3(kNT), 0, s, a);
    if (d == 128) hipLaunchKernelGGL((route_score<uint16_t, 128, MODE>), grid, dim3(kNT), 0, s, a);
  } else {
    if (d == 32) hipLaunchKernelGGL((route_score<float, 32, MODE>), grid, dim3(kNT), 0, s, a);
    if (d == 64) hipLaunchKernelGGL((route_score<float, 64, MODE>), grid, dim3(kNT), 0, s, a);
    if (d == 128) hipLaunchKernelGGL((route_score<float, 128, MODE>), grid, dim3(kNT), 0, s, a);
  }
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
  a.ticket1 = reinterpret_cast<uint32_t*>(base + L.o_t1);
  a.ticket2 = reinterpret_cast<uint32_t*>(base + L.o_t2);
  a.ccount = reinterpret_cast<uint32_t*>(base + L.o_cc);
  a.ghist = reinterpret_cast<uint32_t*>(base + L.o_gh);
  a.info = reinterpret_cast<RowInfo*>(base + L.o_info);
  a.cnt = reinterpret_cast<uint32_t*>(base + L.o_cnt);
  a.coff = reinterpret_cast<uint32_t*>(base + L.o_coff);
  a.keys = reinterpret_cast<uint32_t*>(base + L.o_keys);
  a.cand = reinterpret_cast<uint64_t*>(base + L.o_cand);
  return a;
}

}  // namespace
}  // namespace clsa

using namespace clsa;

extern "C" size_t clsa_route_workspace_size(int B, int M, int d, int64_t n_cap, int k, int cap,
                                            clsa_dtype dt) {
  (void)dt;
  if (!shape_ok(B, M, d, n_cap, cap) || k < 1) return 0;
  return make_layout((int64_t)B * M, n_cap, true).total;
}

extern "C" int clsa_route(const void* q_idx, const void* K_idx, int B, int M, int d,
                          int64_t n_cap, const int32_t* n_ctx, int64_t q_pos0, int k,
                          clsa_dtype dt, int32_t* idx, int32_t* counts, int cap, void* ws,
                          size_t ws_bytes, void* stream) {
  if (dt != CLSA_F32 && dt != CLSA_BF16) return CLSA_ERR_UNSUPPORTED_DTYPE;
  if (!q_idx || !K_idx || !idx || !counts) return CLSA_ERR_INVALID;
  if (!shape_ok(B, M, d, n_cap, cap) || k < 1 || cap < k) return CLSA_ERR_INVALID;
  const int64_t R = (int64_t)B * M;
  const Layout L = make_layout(R, n_cap, true);
  if (!ws || ws_bytes < L.total) return CLSA_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const RouteArgs a = fill_args(L, ws, q_idx, K_idx, B, M, n_cap, n_ctx, q_pos0, k, nullptr,
                                idx, counts, cap);
  if (zero_fill(ws, L.ctrl_end, s) != hipSuccess) return CLSA_ERR_HIP;
  const dim3 grid((unsigned)L.C, (unsigned)R);
  launch_score<kModeTopk>(a, dt, d, grid, s);
  hipLaunchKernelGGL(route_cands, grid, dim3(kNT), 0, s, a);
  hipLaunchKernelGGL(route_compact, grid, dim3(kNT), 0, s, a);
  return hipGetLastError() == hipSuccess ? CLSA_OK : CLSA_ERR_HIP;
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
  if (zero_fill(ws, L.ctrl_end, s) != hipSuccess) return CLSA_ERR_HIP;
  const dim3 grid((unsigned)L.C, (unsigned)R);
  launch_score<kModeThresh>(a, dt, d, grid, s);
  hipLaunchKernelGGL(route_compact, grid, dim3(kNT), 0, s, a);
  return hipGetLastError() == hipSuccess ? CLSA_OK : CLSA_ERR_HIP;
}

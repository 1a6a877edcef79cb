// Block routing: top-k for many query rows of one sequence (a prefill chunk),
// with the score matrix on the matrix cores.
//
// Method: CLSA explainer (ai-papers.net), section "CLSAの仕組み" -- the
// self-decoder picks the top-k KV positions of every query token once; for a
// chunk of M query tokens that is the dense score matrix Q_idx K_idx^T
// (causally masked) followed by a row-wise top-k.  The scores are a real
// dense contraction, so they run on v_mfma_f32_32x32x16_bf16 and the score
// matrix never reaches HBM.
//
//   block_thresh   per group of 16 rows: scores against every ss-th key
//                  (MFMA), each lane keeping per row the largest 16-bit key
//                  prefixes it sees; per row a lower bound of the rho-th
//                  largest sampled score, rho chosen so that, with a
//                  four-sigma margin, at least k keys of the row score that
//                  much.  It becomes the row's filter threshold T.
//   block_filter   the full score matrix in 32x32 MFMA tiles, keys as the A
//                  operand and queries as B, so each lane owns one query
//                  column (two lanes per row, one per key half); a workgroup
//                  streams a key chunk through LDS while each wave keeps one
//                  32-row query slab in registers.  Keys scoring >= T are
//                  appended as (score - T', position) to the row's segment
//                  of the chunk.
//   block_select   per row: the exact top-k among the candidates (lower
//                  positions win ties), written in ascending order.  A row
//                  whose threshold kept fewer than k keys, or more than the
//                  select holds, is redone by an exact rescan (rare).
// All keys of a row are ranked on values computed the same way, so equal key
// rows score exactly equal and the lower position wins.
#include "clsa_common.h"
#include "clsa_rowplan.h"
#include "clsa_select.h"

namespace clsa {
namespace {

constexpr int kNT = kSelNT;        // threads of the thresh/select kernels
constexpr int kFT = 512;           // threads of the filter kernel (8 waves)
constexpr int kSStride = 32;       // sampling stride of the threshold estimate
constexpr int kStageKeys = 64;     // keys per filter step (two 32-key tiles)
constexpr int kSelCap = 6144;      // candidates a select workgroup holds
constexpr int kMaxK = 2048;
constexpr int kMaxSegs = 2048;     // candidate segments (key chunks) per row
constexpr int64_t kMaxKeys = 524288;

// Keys held in LDS by a filter workgroup at a time (16 KB of bf16 keys),
// and keys per candidate segment: a workgroup walks kSubPerChunk of those
// in turn, so a row's segment of one chunk covers 16x as many keys and its
// cache lines fill before they are written back.
constexpr int sub_keys(int d) { return 8192 / d; }
constexpr int kSubPerChunk = 16;
constexpr int chunk_keys(int d) { return kSubPerChunk * sub_keys(d); }
// Filter rows per workgroup (one 32-row slab per wave).  16 KB of keys and
// 64 KB of hit scratch let two workgroups share a CU, four waves per SIMD,
// so one wave's hit extraction overlaps another's matrix work; the 64
// workgroups of an XCD keep their partly filled segment lines (one per row)
// within its 4 MB L2, so they fill before they are written back.
constexpr int kMaxRowsPerGroup = 256;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

struct BlockArgs {
  const uint16_t* q;       // [B][M][d] bf16
  const uint16_t* K;       // [B][n_cap][d] bf16
  const int32_t* n_ctx;    // [B] or null
  int32_t* idx;            // [B][M][cap]
  int32_t* counts;         // [B][M]
  int64_t n_cap, q_pos0;
  int B, M, k, cap;
  int ns_max;              // sampled keys per row (max, <= kThrNs)
  int64_t ss;              // sampling stride (keys)
  int kc;                  // keys per chunk (chunk_keys(d))
  int nchunks;             // key chunks per row
  int rows_pg;             // rows per filter workgroup (multiple of 64)
  int segcap;              // decode rows: candidate entries per chunk and row (row_seg_cap)
  float* thr;              // [R] filter threshold; -inf: every key, +inf: none
  uint32_t* segcnt;        // [R][nchunks] candidates per segment
  uint64_t* seg;           // [R][nchunks][kc]: position | (score - T') << 32
};

CLSA_DEV int64_t row_visible(const BlockArgs& a, int b, int m) {
  int64_t n = a.n_ctx ? (int64_t)a.n_ctx[b] : a.n_cap;
  n = n < 0 ? 0 : (n > a.n_cap ? a.n_cap : n);
  if (a.q_pos0 >= 0) {
    const int64_t lim = a.q_pos0 + m + 1;
    n = n < lim ? n : lim;
  }
  return n;
}

// Operands of a 32-row slab for v_mfma_f32_32x32x16_bf16: lane l holds row
// l%32, dims 16*st + 8*(l/32) .. +7 for k-step st (A and B layouts agree).
template <int D>
CLSA_DEV void load_q_slab(const BlockArgs& a, int b, int m0, bf16x8_t (&qa)[D / 16]) {
  const int lane = lane_id();
  const int m = m0 + lane % 32;
  const bool ok = m < a.M;
#pragma unroll
  for (int st = 0; st < D / 16; ++st) {
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (ok)
      v = *reinterpret_cast<const u32x4_t*>(a.q + ((size_t)b * a.M + m) * D + st * 16 +
                                              8 * (lane / 32));
    qa[st] = __builtin_bit_cast(bf16x8_t, v);
  }
}

// Staged keys in LDS: key n holds P = D/8 16-byte pieces; piece c sits in
// slot c ^ ((n / (16/P)) % P).  LDS serves 16 lanes x 16 bytes per clock
// from 64 banks, so the 16 lanes reading one piece of 16 consecutive keys
// must cover 16 distinct 16-byte bank groups: the keys' rows fix the group
// modulo 16/P, the slot swizzle the rest.
template <int D>
CLSA_DEV int lds_piece(int n, int c) {
  constexpr int P = D / 8;
  constexpr int kShift = P >= 16 ? 0 : (P == 8 ? 1 : 2);
  static_assert(P == 4 || P == 8 || P == 16, "d_idx 32, 64 or 128");
  return n * P + (c ^ ((n >> kShift) & (P - 1)));
}

template <int D>
CLSA_DEV void load_k_tile(const u32x4_t* lds, int t, bf16x8_t (&kb)[D / 16]) {
  const int lane = lane_id();
  const int n = t * 32 + lane % 32;
#pragma unroll
  for (int st = 0; st < D / 16; ++st)
    kb[st] = __builtin_bit_cast(bf16x8_t, lds[lds_piece<D>(n, 2 * st + lane / 32)]);
}

// c + X Y^T over one 32x32 tile (rows of X against rows of Y)
template <int D>
CLSA_DEV f32x16_t tile_mma(const bf16x8_t (&x)[D / 16], const bf16x8_t (&y)[D / 16], f32x16_t c) {
#pragma unroll
  for (int st = 0; st < D / 16; ++st)
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x[st], y[st], c, 0, 0, 0);
  return c;
}

// Exact rank-th largest of the n 32-bit keys get(0 .. n-1), 1 <= rank <= n,
// by three histogram passes over bits 31..21, 20..10 and 9..0.  *left gets
// how many elements equal to the result are needed to reach the rank.
template <class Get>
CLSA_DEV uint32_t select_key_desc(Get get, uint32_t n, uint32_t rank, uint32_t* h, uint32_t* tmp,
                                  uint32_t* bc, uint32_t* left) {
  uint32_t prefix = 0;
#pragma unroll
  for (int p = 0; p < 3; ++p) {
    const int shift = p == 0 ? 21 : (p == 1 ? 10 : 0);
    const uint32_t width = p == 2 ? 1023u : 2047u;
    const uint32_t pmask = p == 0 ? 0u : (p == 1 ? 0xFFE00000u : 0xFFFFFC00u);
    for (int i = threadIdx.x; i < 2048; i += kNT) h[i] = 0u;
    __syncthreads();
    for (uint32_t i = threadIdx.x; i < n; i += kNT) {
      const uint32_t key = get(i);
      if ((key & pmask) == prefix) atomicAdd(&h[(key >> shift) & width], 1u);
    }
    __syncthreads();
    if (p < 2) find_bin_desc<2048>(h, rank, tmp, bc);
    else find_bin_desc<1024>(h, rank, tmp, bc);
    prefix |= bc[0] << shift;
    rank = bc[1];
    __syncthreads();
  }
  *left = rank;
  return prefix;
}

// ------------------------------------------------------------------ thresh
// One workgroup per 16 query rows.  Scores against every a.ss-th key come
// from v_mfma_f32_16x16x32_bf16; as they come out of the accumulator, each
// lane keeps, per row, the 8 largest scores among the samples it sees (an
// insertion chain: slot i becomes the median of slot i-1, slot i and the
// new value) and stores their top-16-bit order-preserving key prefixes.
// The 128 such lists of a row (8 waves x 16 sample lanes, 1024 prefixes) go to LDS,
// and a wave ranks each of its rows' lists: a 1024-bin histogram over their
// actual range and a second pass over the boundary bin give the rho-th
// largest.  The lists are samples, so that prefix is at most the rho-th
// largest sample's, and equal to it unless one list held more than 8 of the
// top rho (rho <= 105 for k <= 2048 here); the threshold is the smallest
// float with that prefix -- never above the sample.  rho is the smallest
// count with rho - 4 sqrt(rho) >= k * ns / n, so at least k keys of the row
// score above the threshold with high probability; rows where it keeps
// fewer (or too many) keys are caught by the select.
constexpr int kThrRows = 16;  // rows per workgroup (<= 16, the MFMA block's rows; a multiple of 4)
constexpr int kThrNs = 4096;  // sampled keys per row at most
constexpr int kThrTiles = 4;  // 16-sample tiles whose loads are in flight together
constexpr int kThrBins = 1024;
constexpr int kThrTop = 8;    // prefixes each lane keeps per row
constexpr int kThrKept = kNT / kWave * 16 * kThrTop;  // kept prefixes per row
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <int D>
__global__ __launch_bounds__(kNT) void block_thresh(BlockArgs a) {
  __shared__ uint16_t kept[kThrRows][kThrKept];
  __shared__ uint32_t wh[kNT / kWave][kThrBins];
  const int m0 = blockIdx.x * kThrRows, b = blockIdx.y;
  const int lane = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);

  // A operand: row m0 + lane%16, dims 32*st + 8*(lane/16) .. +7
  bf16x8_t qa[D / 32];
  {
    const int m = m0 + lane % 16;
#pragma unroll
    for (int st = 0; st < D / 32; ++st) {
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (lane % 16 < kThrRows && m < a.M)
        v = *reinterpret_cast<const u32x4_t*>(a.q + ((size_t)b * a.M + m) * D + 32 * st +
                                                8 * (lane / 16));
      qa[st] = __builtin_bit_cast(bf16x8_t, v);
    }
  }
  // accumulator value j of this lane is row 4*(lane/16) + j, sample lane%16
  int64_t lim[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int m = m0 + 4 * (lane / 16) + j;
    lim[j] = m < a.M ? row_visible(a, b, m) : 0;
  }
  // per row: this lane's largest scores, descending; -inf = none.  The
  // 16-bit key prefix is a monotone map of the score, so the largest
  // prefixes are the prefixes of the largest scores: the lists hold floats
  // (one v_med3_f32 per slot and sample) and are mapped once at the end.
  float t8[4][kThrTop];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < kThrTop; ++i) t8[j][i] = -INFINITY;
  const int ntile = (a.ns_max + 15) / 16;
  for (int t0 = w * kThrTiles; t0 < ntile; t0 += (kNT / kWave) * kThrTiles) {
    bf16x8_t kb[kThrTiles][D / 32];
#pragma unroll
    for (int u = 0; u < kThrTiles; ++u) {
      const int64_t smp = (int64_t)(t0 + u) * 16 + lane % 16;
      const int64_t j = smp * a.ss;
#pragma unroll
      for (int st = 0; st < D / 32; ++st) {
        u32x4_t v = {0u, 0u, 0u, 0u};
        if (t0 + u < ntile && smp < a.ns_max && j < a.n_cap)
          v = *reinterpret_cast<const u32x4_t*>(a.K + ((size_t)b * a.n_cap + j) * D + 32 * st +
                                                  8 * (lane / 16));
        kb[u][st] = __builtin_bit_cast(bf16x8_t, v);
      }
    }
#pragma unroll
    for (int u = 0; u < kThrTiles; ++u) {
      f32x4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < D / 32; ++st)
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[st], kb[u][st], c, 0, 0, 0);
      const int64_t smp = (int64_t)(t0 + u) * 16 + lane % 16;
      const int64_t j = smp * a.ss;
      const bool in = t0 + u < ntile && smp < a.ns_max;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        // a NaN score counts as no sample (fmaxf returns the other operand)
        const float x = (in && j < lim[jj]) ? fmaxf(c[jj], -INFINITY) : -INFINITY;
        // slot i becomes the median of slot i-1, slot i and x (the list is
        // sorted, so that is max(slot i, min(slot i-1, x)))
#pragma unroll
        for (int i = kThrTop - 1; i >= 1; --i)
          t8[jj][i] = __builtin_amdgcn_fmed3f(t8[jj][i - 1], t8[jj][i], x);
        t8[jj][0] = fmaxf(t8[jj][0], x);
      }
    }
  }
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const int rl = 4 * (lane / 16) + jj;
    if (rl < kThrRows) {
      uint16_t* dst = &kept[rl][(w * 16 + lane % 16) * kThrTop];
#pragma unroll
      for (int i = 0; i < kThrTop; ++i)
        dst[i] = t8[jj][i] == -INFINITY ? (uint16_t)0 : (uint16_t)(score_key(t8[jj][i]) >> 16);
    }
  }
  __syncthreads();

  uint32_t* h = wh[w];
  for (int rl = w; rl < kThrRows; rl += kNT / kWave) {
    const int m = m0 + rl;
    if (m >= a.M) break;
    const int r = b * a.M + m;
    const int64_t n_vis = row_visible(a, b, m);
    const int64_t k_eff = a.k < n_vis ? a.k : n_vis;
    if (k_eff >= n_vis) {  // every visible key is selected: no candidates needed
      if (lane == 0) a.thr[r] = INFINITY;
      continue;
    }
    const int ns = (int)((n_vis + a.ss - 1) / a.ss);  // visible samples
    const int rho = sample_rank(n_vis, k_eff, ns);
    // the row's kept prefixes (lane l: entries l, l+64, ...); 0 marks an
    // empty slot (no real key has a zero prefix)
    uint32_t v[kThrKept / kWave];
    uint32_t nk = 0;
#pragma unroll
    for (int u = 0; u < kThrKept / kWave; ++u) {
      v[u] = kept[rl][lane + u * kWave];
      nk += v[u] != 0u ? 1u : 0u;
    }
    if (rho > ns || (uint32_t)rho > wave_sum_u32(nk)) {
      // too few samples to bound the k-th score: keep every key
      if (lane == 0) a.thr[r] = -INFINITY;
      continue;
    }
    const uint32_t kth =
        wave_kth_u16(v, [&](int u) { return v[u] != 0u; }, (uint32_t)rho, h);
    // smallest float of the 16-bit bucket: never above the sample
    if (lane == 0) a.thr[r] = key_to_float(kth << 16);
  }
}

// Rows whose keys no other row shares (a decode step: one query per
// sequence), sampled as row_plan says: ceil(ns / kNT) workgroups score the
// samples, one per thread, on the VALU (v_dot2_f32_bf16 against the row's
// query; a single query row has no matrix shape to give the matrix cores),
// and store their 16-bit key prefixes -- each wave's p.top largest when
// the plan is compact, else all of them -- for the score pass, which ranks
// them (rank_row_samples).  The sample scores only set a threshold that the
// select checks, so their summation order does not matter.
constexpr int kRowNs = kRowSamples;
constexpr int kRowSampleWG = kRowNs / kNT;  // one sample per thread

template <int D>
__global__ __launch_bounds__(kNT) void row_sample(BlockArgs a, uint16_t* samp) {
  const int r = blockIdx.y, b = r / a.M, m = r % a.M;
  const int lane = lane_id(), w = threadIdx.x / kWave;
  const int64_t n_vis = row_visible(a, b, m);
  const int64_t k_eff = a.k < n_vis ? a.k : n_vis;
  if (k_eff >= n_vis) return;  // the select takes every visible key
  const RowPlan p = row_plan(n_vis, k_eff);
  const int s0 = blockIdx.x * kNT + w * kWave;  // the wave's 64 samples, one per lane
  if (p.rho > p.ns || s0 >= p.ns) return;
  uint16_t* row = samp + (size_t)r * kRowNs;

  const int smp = s0 + lane;
  u32x4_t kv[D / 8];
  const u32x4_t* kp = reinterpret_cast<const u32x4_t*>(
      a.K + ((size_t)b * a.n_cap + (size_t)((int64_t)(smp < p.ns ? smp : 0) * n_vis / p.ns)) * D);
#pragma unroll
  for (int st = 0; st < D / 8; ++st) kv[st] = kp[st];
  const u32x4_t* qp = reinterpret_cast<const u32x4_t*>(a.q + (size_t)r * D);
  float acc = 0.f;
#pragma unroll
  for (int st = 0; st < D / 8; ++st) {
    const u32x4_t qv = qp[st];
    acc = dot2(kv[st][0], qv[0], acc);
    acc = dot2(kv[st][1], qv[1], acc);
    acc = dot2(kv[st][2], qv[2], acc);
    acc = dot2(kv[st][3], qv[3], acc);
  }
  // samples past ns count as 0, below every real prefix
  uint32_t key = smp < p.ns ? score_key(acc) >> 16 : 0u;
  if (p.compact) {
    // the wave's p.top largest: take the maximum, knock one copy out
    for (int t = 0; t < p.top; ++t) {
      const uint32_t mx = wave_max_u32(key);
      const uint64_t has = __ballot(key == mx);
      if (lane == __ffsll((unsigned long long)has) - 1) key = 0u;
      if (lane == 0) row[(s0 / kWave) * p.top + t] = (uint16_t)mx;
    }
  } else if (smp < p.ns) {
    row[smp] = (uint16_t)key;
  }
}

// ------------------------------------------------------------------ filter
// Each workgroup walks one chunk of chunk_keys(d) keys, sub_keys(d) at a
// time in LDS, and each of its 8 waves keeps one 32-row query slab in
// registers for the whole chunk: no barrier inside a sub-chunk, and the
// chunk is read from HBM once per workgroup.
//
// A last MFMA k-step against a constant column subtracts the row's
// threshold inside the accumulator: dd = score - T', with T' the threshold
// rounded down to bf16 (still a lower bound, so nothing is lost).  The sign
// bits of a step's 32 values per lane pack into one hit mask with one
// v_alignbit each; lanes with hits spill their 32 values to LDS scratch and
// up to four hits per lane per pass are appended as (dd, position) to the
// row's segment in HBM, the two lanes of a row one after the other.  Rows
// that keep every key (threshold -inf) and tiles crossing a row's
// visibility limit take explicit compares instead.
constexpr int kScrStride = 32;  // scratch words per lane: the step's 32 values
// A wave's scratch is value-major: value i of lane l sits in word
// i * 64 + l, so each lane stays in its own bank and the reads of hits at
// different value indices never conflict.  (Lane-major 16-byte pieces made
// those reads conflict and cost the filter 2 us.)

// bf16 bits of -x, with x first rounded down to bf16 (toward -inf)
CLSA_DEV uint16_t neg_bf16_floor(float x) {
  uint32_t u = __float_as_uint(x);
  if (x == 0.f) return 0;  // +0: keeps dd = +0 for a zero score
  const uint32_t t = u & 0xffff0000u;
  u = (t != u && (u >> 31)) ? t + 0x10000u : t;  // negative: away from zero
  return (uint16_t)((u ^ 0x80000000u) >> 16);
}

struct SlabState {
  bf16x8_t tq;      // k-step operand: -T' in dim 0 (lanes < 32)
  float lo;         // 0, or -inf when the row keeps every key
  int32_t lim;      // keys visible to the lane's row
  int32_t lim_min;  // min over the slab (wave-uniform)
  bool sign_ok;     // every row of the slab has a finite threshold (uniform)
  uint64_t* segp;   // the row's segment of this chunk in HBM
  uint32_t gcnt;    // entries written there (both lanes of the row)
};

// One step (two 32-key tiles) of one slab: the 32 values of this lane's
// query, value i being key jl0 + 2*(i & 28) + (i & 3).  Returns the hit
// mask, bit i for value i.
template <bool CHECK>
CLSA_DEV uint32_t stage_hits(const f32x16_t& x0, const f32x16_t& x1, const SlabState& st,
                             int32_t jl0) {
  uint32_t m = 0;  // after the chain, bit i is the sign of value i (1: miss)
  // opaque copy: keeps the compiler from hoisting the compare path's
  // position arithmetic into the fast path
  if (CHECK) asm volatile("" : "+v"(jl0));
#pragma unroll
  for (int i = 31; i >= 0; --i) {
    const float x = i < 16 ? x0[i] : x1[i - 16];
    if (CHECK) {
      const int32_t j = jl0 + 2 * (i & 28) + (i & 3);
      const bool hit = x >= st.lo && j < st.lim;
      m = __builtin_amdgcn_alignbit(m, hit ? 0u : 0x80000000u, 31);
    } else {
      m = __builtin_amdgcn_alignbit(m, __float_as_uint(x), 31);
    }
  }
  return ~m;
}

// Spill the step's values of lanes with hits to the wave's scratch (each
// 32-key tile only where it holds a hit), then append the hits (dd, position) to the
// row's segment, up to four per lane per pass so that each pass waits on
// LDS once.  Value i of a lane is key jl0 + i + (i & 28).
CLSA_DEV void stage_emit(const f32x16_t& x0, const f32x16_t& x1, uint32_t hits, SlabState& st,
                         int32_t jl0, float* scr) {
  const int lane = lane_id();
  if ((hits & 0xffffu) != 0u) {
#pragma unroll
    for (int i = 0; i < 16; ++i) scr[i * kWave + lane] = x0[i];
  }
  if ((hits >> 16) != 0u) {
#pragma unroll
    for (int i = 0; i < 16; ++i) scr[(16 + i) * kWave + lane] = x1[i];
  }
  while (__ballot(hits != 0u) != 0) {
    int idx[4];
    float dv[4];
    uint32_t h = hits;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      idx[q] = h != 0u ? __builtin_ctz(h) : 0;
      h &= h - 1u;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) dv[q] = scr[idx[q] * kWave + lane];
    const uint32_t n = __popc(hits) - __popc(h);  // hits taken this pass (<= 4)
    // lanes l and l+32 hold the same row: one stream, the upper lane after
    // the lower one.  Swapping the wave's halves gives every lane the lower
    // lane's count (sw2[0] in the upper half) and the pair's total.
    const auto sw2 = __builtin_amdgcn_permlane32_swap(n, n, false, false);
    const uint32_t pair_total = sw2[0] + sw2[1];
    const uint32_t at = st.gcnt + (lane >= 32 ? sw2[0] : 0u);
    uint32_t pw[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) pw[q] = (uint32_t)(jl0 + idx[q] + (idx[q] & 28));
    // exactly the pass's n entries (the partner lane's follow them)
    uint64_t* dst = st.segp + at;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if ((uint32_t)q < n) dst[q] = ((uint64_t)__float_as_uint(dv[q]) << 32) | pw[q];
    st.gcnt += pair_total;
    hits = h;
  }
}

// Query operands and per-row state of the slab at rows m0 .. m0+31
template <int D>
CLSA_DEV void load_slab(const BlockArgs& a, int b, int m0, int ch, bf16x8_t (&qb)[D / 16],
                        SlabState& st) {
  const int lane = lane_id();
  const int m = m0 + lane % 32;
  const bool ok = m < a.M;
  load_q_slab<D>(a, b, m0, qb);
  const float T = ok ? a.thr[(size_t)b * a.M + m] : INFINITY;
  const bool all = T == -INFINITY;
  st.tq = __builtin_bit_cast(
      bf16x8_t, u32x4_t{lane < 32 ? (uint32_t)(all ? 0u : neg_bf16_floor(T)) : 0u, 0u, 0u, 0u});
  st.lo = all ? -INFINITY : 0.f;
  st.lim = ok ? (int32_t)row_visible(a, b, m) : 0;
  st.lim_min = (m0 + 31 < a.M) ? (int32_t)row_visible(a, b, m0) : 0;
  st.sign_ok = __ballot(all) == 0;
  const size_t sg = ((size_t)b * a.M + (ok ? m : 0)) * a.nchunks + ch;
  st.segp = a.seg + sg * (size_t)a.kc;
  st.gcnt = 0;
}

// grid: (nchunks, ceil(M / rows_pg), B); rows_pg <= kMaxRowsPerGroup, a
// multiple of 32.  Wave w owns the slab at rows r_lo + 32 w and keeps its
// operands and segment counts across the sub-chunks.
template <int D>
__global__ __launch_bounds__(kFT) __attribute__((amdgpu_waves_per_eu(D <= 64 ? 4 : 2, 8)))
void block_filter(BlockArgs a) {
  constexpr int KS = sub_keys(D);
  constexpr int P = D / 8;  // 16-byte pieces per key
  __shared__ u32x4_t kc[KS * P];
  __shared__ __attribute__((aligned(16))) float scratch[kFT / kWave][kWave * kScrStride];
  const int ch = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int lane = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int r_lo = g * a.rows_pg;
  const int r_hi = r_lo + a.rows_pg < a.M ? r_lo + a.rows_pg : a.M;
  const int64_t vis_hi = row_visible(a, b, r_hi - 1);  // visibility grows with m
  float* scr = &scratch[w][0];  // the wave's scratch, value-major
  const bf16x8_t kone =  // constant operand of the threshold k-step: 1.0 in dim 0
      __builtin_bit_cast(bf16x8_t, u32x4_t{lane < 32 ? 0x3f80u : 0u, 0u, 0u, 0u});
  const int m0 = r_lo + 32 * w;
  const bool active = m0 < r_hi;  // wave-uniform
  bf16x8_t qb[D / 16];
  SlabState st;
  int64_t vis_slab = 0;  // keys visible to the slab's last row
  if (active) {
    load_slab<D>(a, b, m0, ch, qb, st);
    vis_slab = row_visible(a, b, (m0 + 31 < r_hi ? m0 + 31 : r_hi - 1));
  }

  for (int sc = 0; sc < kSubPerChunk; ++sc) {
    const int64_t key_lo = (int64_t)ch * a.kc + (int64_t)sc * KS;
    const int64_t key_hi = key_lo + KS < vis_hi ? key_lo + KS : vis_hi;
    if (key_lo >= key_hi) break;  // uniform: nothing further is visible
    if (sc > 0) __syncthreads();  // the previous sub-chunk is no longer read
    // the sub-chunk's keys, zeros at or beyond key_hi
    {
      constexpr int kPer = KS * P / kFT;
      u32x4_t v[kPer];
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        const int i = threadIdx.x + u * kFT;
        const int64_t j = key_lo + i / P;
        v[u] = u32x4_t{0u, 0u, 0u, 0u};
        if (j < key_hi)
          v[u] = *reinterpret_cast<const u32x4_t*>(a.K + ((size_t)b * a.n_cap + j) * D + (i % P) * 8);
      }
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        const int i = threadIdx.x + u * kFT;
        kc[lds_piece<D>(i / P, i % P)] = v[u];
      }
    }
    __syncthreads();
    if (!active) continue;

    const int64_t hi_p = key_hi < vis_slab ? key_hi : vis_slab;
    const int nstage = hi_p > key_lo ? (int)((hi_p - key_lo + kStageKeys - 1) / kStageKeys) : 0;
    for (int sidx = 0; sidx < nstage; ++sidx) {
      const int32_t js = (int32_t)(key_lo + (int64_t)sidx * kStageKeys);  // step start
      const int32_t jl0 = js + 4 * (lane / 32);
      bf16x8_t kb0[D / 16], kb1[D / 16];
      load_k_tile<D>(kc, 2 * sidx, kb0);
      load_k_tile<D>(kc, 2 * sidx + 1, kb1);
      // all of the step's key reads go out before its first MFMA (left to
      // itself the scheduler feeds each MFMA its own just-in-time read, one
      // LDS round trip per k-step)
      __builtin_amdgcn_sched_barrier(0);
      // rows: keys, columns: queries; the last k-step subtracts T'
      f32x16_t x0 = tile_mma<D>(kb0, qb, f32x16_t{});
      f32x16_t x1 = tile_mma<D>(kb1, qb, f32x16_t{});
      x0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kone, st.tq, x0, 0, 0, 0);
      x1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kone, st.tq, x1, 0, 0, 0);
      // wave-uniform: a scalar branch keeps the compare path out of the
      // fast one
      const bool fast = __builtin_amdgcn_readfirstlane(
                            (int)(st.sign_ok && js + kStageKeys <= st.lim_min)) != 0;
      uint32_t hits;
      if (fast) hits = stage_hits<false>(x0, x1, st, jl0);
      else hits = stage_hits<true>(x0, x1, st, jl0);
      stage_emit(x0, x1, hits, st, jl0, scr);
    }
  }
  // every (row, chunk) of the group gets its count, zero when it saw nothing
  if (active) {
    const int m = m0 + lane % 32;
    if (m < r_hi && lane < 32) a.segcnt[((size_t)b * a.M + m) * a.nchunks + ch] = st.gcnt;
  }
}

// ------------------------------------------------------------------ select
// q . K_idx[j] for the exact rescan; every key of the row uses this order
template <int D>
CLSA_DEV float row_score(const BlockArgs& a, int b, const float* qf, int64_t j) {
  const uint16_t* kr = a.K + ((size_t)b * a.n_cap + j) * D;
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < D / 8; ++c) {
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(kr + c * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      s = fmaf(qf[c * 8 + 2 * e], bf16_lo(v[e]), s);
      s = fmaf(qf[c * 8 + 2 * e + 1], bf16_hi(v[e]), s);
    }
  }
  return s;
}

// Exact top-k of one row from recomputed scores: a radix select of the k-th
// key, then the positions in order (keys above it and the first `left`
// equal to it).
template <int D>
CLSA_DEV void exact_rescan(const BlockArgs& a, int b, int m, int64_t n_vis, int64_t k_eff,
                           int32_t* out, uint32_t* h, uint32_t* tmp, uint32_t* bc, uint32_t* wcnt) {
  const int tid = threadIdx.x;
  float qf[D];
  {
    const uint16_t* qr = a.q + ((size_t)b * a.M + m) * D;
#pragma unroll
    for (int e = 0; e < D; ++e) qf[e] = __uint_as_float((uint32_t)qr[e] << 16);
  }
  uint32_t left;
  const uint32_t kstar = select_key_desc(
      [&](uint32_t i) { return score_key(row_score<D>(a, b, qf, i)); }, (uint32_t)n_vis,
      (uint32_t)k_eff, h, tmp, bc, &left);
  uint32_t run = 0, eq_seen = 0;
  for (int64_t j0 = 0; j0 < n_vis; j0 += kNT) {
    const int64_t j = j0 + tid;
    const uint32_t key = j < n_vis ? score_key(row_score<D>(a, b, qf, j)) : 0u;
    const bool eq = j < n_vis && key == kstar;
    uint32_t eq_tot;
    const uint32_t eq_rank = eq_seen + block_rank<kNT>(eq, wcnt, &eq_tot);
    const bool take = j < n_vis && (key > kstar || (eq && eq_rank < left));
    uint32_t tot;
    const uint32_t slot = run + block_rank<kNT>(take, wcnt, &tot);
    if (take) out[slot] = (int32_t)j;
    run += tot;
    eq_seen += eq_tot;
  }
}


// Exclusive scan of n values in[] into out[] (in == out allowed); returns
// the total.  Every thread of the block must call it.
CLSA_DEV uint32_t block_excl_scan_arr(const uint32_t* in, uint32_t* out, int n, uint32_t* tmp,
                                      uint32_t* bc) {
  uint32_t run = 0;
  for (int i0 = 0; i0 < n; i0 += kNT) {
    const int i = i0 + (int)threadIdx.x;
    const uint32_t v = i < n ? in[i] : 0u;
    const uint32_t incl = block_incl_scan<kNT>(v, tmp);
    if (i < n) out[i] = run + incl - v;
    if (threadIdx.x == kNT - 1) bc[0] = incl;
    __syncthreads();
    run += bc[0];
    __syncthreads();
  }
  return run;
}

// One workgroup per row.  Each thread holds at most kPerT candidates in
// registers (every kNT-th one); the row's selection is marked in a bitmap
// over its key positions (dynamic LDS, one bit per position) and written
// out in position order from a popcount prefix over the bitmap's words.
constexpr int kPerT = kSelCap / kNT;

// Bitmap words each select thread owns (contiguous, a multiple of 4 so they
// are read 16 bytes at a time); the bitmap covers kNT times that many words
// and is followed by a 16-bit prefix per word.
__host__ __device__ inline int select_words_per_thread(int64_t n_cap) {
  const int64_t w = ceil_div64(ceil_div64(n_cap, 32), kNT);
  return (int)((w + 3) / 4 * 4);
}
inline size_t select_lds_bytes(int64_t n_cap) {
  return select_bitmap_lds_bytes(select_words_per_thread(n_cap));
}

// The row's candidates sit in segments, one per key chunk, with
// segcnt[r][c] entries each.  Block routing (ROWSEG false): a.nchunks
// segments of a.kc entries, one per chunk of a.kc keys.  Decode rows
// (ROWSEG true): a row owns a.nchunks x a.segcap entries, shared by its
// visible chunks of a.kc keys (row_seg_cap); a count above that share means
// the segment overflowed, and the row is rescanned.
template <int D, bool ROWSEG>
__global__ __launch_bounds__(kNT) void block_select(BlockArgs a) {
  extern __shared__ u32x4_t bitmap4[];  // select_lds_bytes(n_cap): bitmap, then word prefixes
  __shared__ uint32_t segoff[kMaxSegs + 1];
  __shared__ SelScratch S;
  __shared__ uint32_t wcnt[kNT / kWave];

  const int r = blockIdx.x;
  const int b = r / a.M, m = r % a.M;
  const int tid = threadIdx.x;
  const int64_t n_vis = row_visible(a, b, m);
  const int64_t k_eff = a.k < n_vis ? a.k : n_vis;
  int32_t* out = a.idx + (size_t)r * a.cap;
  if (tid == 0) a.counts[r] = (int32_t)k_eff;
  for (int64_t i = k_eff + tid; i < a.cap; i += kNT) out[i] = -1;
  if (k_eff >= n_vis) {
    for (int64_t i = tid; i < n_vis; i += kNT) out[i] = (int32_t)i;
    return;
  }
  // the selection bitmap is cleared now; the barriers of the k-th search
  // order it before the marking
  const int wpt = select_words_per_thread(a.n_cap);  // bitmap words per thread, contiguous
  const int w0 = tid * wpt;
  for (int i = w0; i < w0 + wpt; i += 4) bitmap4[i / 4] = u32x4_t{0u, 0u, 0u, 0u};

  // offsets of the row's segments (one per key chunk)
  const int nseg = ROWSEG ? (int)ceil_div64(n_vis, a.kc) : a.nchunks;
  const uint32_t half =  // segment capacity
      ROWSEG ? row_seg_cap(a.nchunks, a.segcap, a.kc, nseg) : (uint32_t)a.kc;
  const uint32_t* cnt_row = a.segcnt + (size_t)r * a.nchunks;
  const uint32_t n_c = block_excl_scan_arr(cnt_row, segoff, nseg, S.tmp, S.bc);
  bool over = false;
  if constexpr (ROWSEG)
    for (int i = tid; i < nseg; i += kNT) over = over || cnt_row[i] > half;
  if (tid == 0) segoff[nseg] = n_c;
  const bool overflow = __syncthreads_or(over ? 1 : 0) != 0;

  if (n_c < (uint32_t)k_eff || n_c > (uint32_t)kSelCap || overflow) {
    exact_rescan<D>(a, b, m, n_vis, k_eff, out, S.h, S.tmp, S.bc, wcnt);
    return;
  }

  // thread t holds the contiguous run of candidates [t * per, t * per + cnt)
  // of the row's concatenated segments.  One binary-lifting search over the
  // offsets finds the segment of the run's first element (the last segment
  // starting at or before it); the rest of the run walks forward from there,
  // passing a segment end at most a few times.  (A search per element, all
  // kPerT in step, cost the kernel a third of its vector instructions.)
  const uint32_t per = (n_c + kNT - 1) / kNT;  // <= kPerT: n_c <= kSelCap
  const uint32_t e0 = (uint32_t)tid * per;
  const int cnt = e0 < n_c ? (int)(n_c - e0 < per ? n_c - e0 : per) : 0;
  uint32_t key[kPerT], pos[kPerT];
  {
    int c = 0;
    if (cnt > 0) {
      int step = 1;
      while (2 * step < nseg) step *= 2;
      for (; step > 0; step >>= 1) {
        const int t = c + step;
        c = segoff[t < nseg ? t : nseg] <= e0 ? t : c;  // segoff[nseg] = n_c: never taken
      }
    }
    // element e of segment c sits at c * half + (e - segoff[c]) = e + delta
    uint32_t start = segoff[c], next = segoff[c + 1];  // c < nseg
    uint32_t delta = (uint32_t)c * half - start;
    uint32_t off[kPerT];
#pragma unroll
    for (int u = 0; u < kPerT; ++u) {
      const uint32_t e = e0 + (uint32_t)u;
      if (u < cnt)
        while (next <= e) {  // ends: segoff[nseg] = n_c > e
          ++c;
          delta += half - (next - start);
          start = next;
          next = segoff[c + 1];
        }
      off[u] = e + delta;
    }
    const uint64_t* rowseg =
        a.seg + (size_t)r * (ROWSEG ? (size_t)a.nchunks * a.segcap : (size_t)nseg * half);
    uint64_t e[kPerT];
#pragma unroll
    for (int u = 0; u < kPerT; ++u) e[u] = u < cnt ? rowseg[off[u]] : 0ull;
#pragma unroll
    for (int u = 0; u < kPerT; ++u) {
      key[u] = score_key(__uint_as_float((uint32_t)(e[u] >> 32)));
      pos[u] = (uint32_t)e[u];
    }
  }

  select_emit<kPerT>(key, pos, cnt, (uint32_t)k_eff, S, bitmap4, wpt, out);
}

template <int D>
void launch_block(const BlockArgs& a, hipStream_t s) {
  const int R = a.B * a.M;
  hipLaunchKernelGGL(block_thresh<D>, dim3((unsigned)((a.M + kThrRows - 1) / kThrRows), (unsigned)a.B),
                     dim3(kNT), 0, s, a);
  hipLaunchKernelGGL(block_filter<D>,
                     dim3((unsigned)a.nchunks, (unsigned)((a.M + a.rows_pg - 1) / a.rows_pg),
                          (unsigned)a.B),
                     dim3(kFT), 0, s, a);
  hipLaunchKernelGGL((block_select<D, false>), dim3((unsigned)R), dim3(kNT),
                     select_lds_bytes(a.n_cap), s, a);
}

struct BlockLayout {
  int ns_max, kc, nchunks;
  int64_t ss;
  size_t o_thr, o_cnt, o_seg, total;
};

BlockLayout block_layout(int64_t R, int d, int64_t n_cap) {
  BlockLayout L{};
  L.ss = kSStride * ceil_div64(n_cap, (int64_t)kSStride * kThrNs);
  L.ns_max = (int)ceil_div64(n_cap, L.ss);
  L.kc = chunk_keys(d);
  L.nchunks = (int)ceil_div64(n_cap, L.kc);
  size_t o = 0;
  L.o_thr = o; o = align_up(o + (size_t)R * 4, 256);
  L.o_cnt = o; o = align_up(o + (size_t)R * L.nchunks * 4, 256);
  L.o_seg = o; o = align_up(o + (size_t)R * L.nchunks * L.kc * 8, 256);
  L.total = o;
  return L;
}

}  // namespace

// ------------------------------------------------------------------- host
bool block_route_applies(int M, int d, int64_t n_cap, int k, clsa_dtype dt) {
  if (dt != CLSA_BF16 || M < 64 || k > kMaxK) return false;
  if (d != 32 && d != 64 && d != 128) return false;
  return n_cap <= kMaxKeys && ceil_div64(n_cap, chunk_keys(d)) <= kMaxSegs;
}

size_t block_route_workspace(int B, int M, int d, int64_t n_cap) {
  return block_layout((int64_t)B * M, d, n_cap).total;
}

int block_route(const void* q_idx, const void* K_idx, int B, int M, int d, int64_t n_cap,
                const int32_t* n_ctx, int64_t q_pos0, int k, int32_t* idx, int32_t* counts,
                int cap, void* ws, hipStream_t s) {
  const BlockLayout L = block_layout((int64_t)B * M, d, n_cap);
  char* base = static_cast<char*>(ws);
  BlockArgs a{};
  a.q = static_cast<const uint16_t*>(q_idx);
  a.K = static_cast<const uint16_t*>(K_idx);
  a.n_ctx = n_ctx;
  a.idx = idx;
  a.counts = counts;
  a.n_cap = n_cap;
  a.q_pos0 = q_pos0 < 0 ? -1 : q_pos0;
  a.B = B;
  a.M = M;
  a.k = k;
  a.cap = cap;
  a.ns_max = L.ns_max;
  a.ss = L.ss;
  a.kc = L.kc;
  a.nchunks = L.nchunks;
  // rows per filter workgroup: enough workgroups to cover the chip once,
  // in multiples of a 32-row slab
  const int64_t want_groups = ceil_div64(256, (int64_t)L.nchunks * B);
  int64_t rows_pg = ceil_div64(M, want_groups < 1 ? 1 : want_groups);
  rows_pg = (rows_pg + 31) / 32 * 32;
  a.rows_pg = (int)(rows_pg < kMaxRowsPerGroup ? rows_pg : kMaxRowsPerGroup);
  a.thr = reinterpret_cast<float*>(base + L.o_thr);
  a.segcnt = reinterpret_cast<uint32_t*>(base + L.o_cnt);
  a.seg = reinterpret_cast<uint64_t*>(base + L.o_seg);
  if (d == 32) launch_block<32>(a, s);
  else if (d == 64) launch_block<64>(a, s);
  else launch_block<128>(a, s);
  return hipGetLastError() == hipSuccess ? CLSA_OK : CLSA_ERR_HIP;
}

// Few query rows per sequence (decode): the threshold and the select of
// block routing around a streaming score pass (clsa_route.hip) that writes
// the candidates of each key chunk into that chunk's segment.
bool seg_route_applies(int /* M: every row count below block routing's qualifies */, int d,
                       int64_t n_cap, int k, clsa_dtype dt) {
  if (dt != CLSA_BF16 || k > kMaxK) return false;
  if (d != 32 && d != 64 && d != 128) return false;
  return n_cap <= kMaxKeys;
}

namespace {
BlockArgs seg_args(const void* q_idx, const void* K_idx, int B, int M, int64_t n_cap,
                   const int32_t* n_ctx, int64_t q_pos0, int k) {
  BlockArgs a{};
  a.q = static_cast<const uint16_t*>(q_idx);
  a.K = static_cast<const uint16_t*>(K_idx);
  a.n_ctx = n_ctx;
  a.n_cap = n_cap;
  a.q_pos0 = q_pos0 < 0 ? -1 : q_pos0;
  a.B = B;
  a.M = M;
  a.k = k;
  return a;
}
}  // namespace

void seg_route_sample(const void* q_idx, const void* K_idx, int B, int M, int d, int64_t n_cap,
                      const int32_t* n_ctx, int64_t q_pos0, int k, uint16_t* samp, hipStream_t s) {
  BlockArgs a = seg_args(q_idx, K_idx, B, M, n_cap, n_ctx, q_pos0, k);
  const dim3 grid((unsigned)kRowSampleWG, (unsigned)(B * M));
  if (d == 32) hipLaunchKernelGGL(row_sample<32>, grid, dim3(kNT), 0, s, a, samp);
  else if (d == 64) hipLaunchKernelGGL(row_sample<64>, grid, dim3(kNT), 0, s, a, samp);
  else hipLaunchKernelGGL(row_sample<128>, grid, dim3(kNT), 0, s, a, samp);
}

void seg_route_select(const void* q_idx, const void* K_idx, int B, int M, int d, int64_t n_cap,
                      const int32_t* n_ctx, int64_t q_pos0, int k, int32_t* idx, int32_t* counts,
                      int cap, int chunk_keys, int nchunks, int segcap, uint32_t* segcnt,
                      uint64_t* seg, hipStream_t s) {
  BlockArgs a = seg_args(q_idx, K_idx, B, M, n_cap, n_ctx, q_pos0, k);
  a.idx = idx;
  a.counts = counts;
  a.cap = cap;
  a.kc = chunk_keys;
  a.nchunks = nchunks;
  a.segcap = segcap;
  a.segcnt = segcnt;
  a.seg = seg;
  const dim3 grid((unsigned)(B * M));
  const size_t lds = select_lds_bytes(n_cap);
  if (d == 32) hipLaunchKernelGGL((block_select<32, true>), grid, dim3(kNT), lds, s, a);
  else if (d == 64) hipLaunchKernelGGL((block_select<64, true>), grid, dim3(kNT), lds, s, a);
  else hipLaunchKernelGGL((block_select<128, true>), grid, dim3(kNT), lds, s, a);
}

}  // namespace clsa

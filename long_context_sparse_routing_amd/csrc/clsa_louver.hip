// Louver index: threshold (half-space) selection that checks only the keys
// whose cluster can hold a score >= tau.
//
// Method: Louver summary (gist.science, arXiv 2605.06763), section
// "2. Louver インデックス" -- the key space is cut into S contiguous
// subspaces; in each, a balanced PCA tree groups the keys into clusters of
// at most r; each cluster has a bounding ball; a query prunes the clusters
// whose ball misses its half-space and checks the rest exactly; keys that
// arrive while decoding wait in a buffer and are clustered into a new part
// of the index when it fills.  Section "クエリアルゴリズム" -- Query 1
// prunes each subspace with its own threshold, Query 2 (TA) scans clusters
// in descending bound with one global threshold until a stopping rule
// holds.  Both have no false negatives.
//
// Build (one segment = a tree over key positions [a, b), all sequences):
//   lv_split    one workgroup per tree node of one level: mean and principal
//               axis of a sample of the node's keys (power iteration), the
//               projection of every member, an exact radix select of the
//               node's median and a stable partition of its slots into the
//               two children.  One launch per level.
//   lv_leaves   one wave per cluster: the members' mean rounded to bf16 is
//               the ball's center; the radius is measured from that rounded
//               center, so the ball is exact for the center it stores.
// Query (one query row per sequence, bf16 keys):
//   lv_bounds   per cluster and subspace the upper bound <q_s, c> + rho |q_s|
//               plus a rounding margin, and per subspace its maximum.
//   lv_ta_depth (Query 2) per row and segment: each subspace's bounds sorted
//               in LDS; the stop depth t*; the bound at rank t* - 1 becomes
//               the subspace's cut.
//   lv_scan     one wave per cluster (of subspace 0 for Query 1, of every
//               subspace for Query 2): skip it when its bound fails, else
//               check its members -- Query 1 first tests the member's
//               clusters in the other subspaces -- and mark keys scoring
//               >= tau in a per-row bitmap over positions.
//   lv_buffer   exact check of the positions past the index (the buffer).
//   lv_compact  the bitmap's positions in ascending order, the true count.
// Scores are fp32 sums of exact bf16 products compared with tau in fp32,
// as in clsa_route_threshold; a cluster is pruned only when its bound plus a
// margin far above fp32 rounding (1e-4 relative) is below the threshold.
#include "clsa_common.h"

namespace clsa {
namespace {

constexpr int kLvMaxSegs = 16;
constexpr int kSplitThreads = 1024;
constexpr int kLvSampleFloats = 16384;  // sampled key components per node (64 KB)
constexpr int kPowerIters = 6;
constexpr int kScanWaves = 4;

struct LvIndex {
  int32_t* perm;       // [B][S][n_max]  slot -> position
  uint16_t* cid;       // [B][S][n_max]  position -> cluster (S > 1)
  uint16_t* centers;   // [B][S][C_max][ds] bf16
  float* radius;       // [B][S][C_max]
  int32_t* cl_begin;   // [C_max + 1]     first slot of each cluster
};

struct LvLayout {
  int64_t n_max;
  int C_max;
  size_t o_perm, o_cid, o_cent, o_rad, o_beg, total;
};

LvLayout lv_layout(int B, int d, int64_t n_max, int S, int r) {
  LvLayout L{};
  L.n_max = n_max;
  L.C_max = (int)(2 * ceil_div64(n_max, r) + kLvMaxSegs);
  const int ds = d / S;
  size_t o = 0;
  L.o_perm = o; o = align_up(o + (size_t)B * S * n_max * 4, 256);
  L.o_cid = o; o = align_up(o + (S > 1 ? (size_t)B * S * n_max * 2 : 0), 256);
  L.o_cent = o; o = align_up(o + (size_t)B * S * L.C_max * ds * 2, 256);
  L.o_rad = o; o = align_up(o + (size_t)B * S * L.C_max * 4, 256);
  L.o_beg = o; o = align_up(o + (size_t)(L.C_max + 1) * 4, 256);
  L.total = o;
  return L;
}

LvIndex lv_index(void* base, const LvLayout& L) {
  char* p = static_cast<char*>(base);
  LvIndex x;
  x.perm = reinterpret_cast<int32_t*>(p + L.o_perm);
  x.cid = reinterpret_cast<uint16_t*>(p + L.o_cid);
  x.centers = reinterpret_cast<uint16_t*>(p + L.o_cent);
  x.radius = reinterpret_cast<float*>(p + L.o_rad);
  x.cl_begin = reinterpret_cast<int32_t*>(p + L.o_beg);
  return x;
}

// fewest levels h with ceil(n / 2^h) <= r
int tree_levels(int64_t n, int r) {
  int h = 0;
  while (ceil_div64(n, (int64_t)1 << h) > r) ++h;
  return h;
}

// ================================================================= build
struct SplitArgs {
  const uint16_t* K;   // [B][n_cap][d]
  int64_t n_cap;
  int d, S, ds;
  int64_t a, n;        // segment start, size
  int level;
  const int32_t* pin;  // [B*S][n] slot -> position (nullptr: slot t is position a + t)
  int32_t* pout;       // [B*S][pout_stride] written at slot offsets
  int64_t pout_stride, pout_off;
  uint32_t* keys;      // [B*S][n] projection keys of the level (scratch)
};

CLSA_DEV int32_t slot_pos(const SplitArgs& a, int bs, int64_t t) {
  return a.pin ? a.pin[(size_t)bs * a.n + t] : (int32_t)(a.a + t);
}

// sub-vector of position p, subspace s, component e (bf16 -> float)
CLSA_DEV const uint16_t* sub_row(const SplitArgs& a, int b, int s, int32_t p) {
  return a.K + ((size_t)b * a.n_cap + p) * a.d + (size_t)s * a.ds;
}

// ascending order of 32-bit keys: the bin of the rank-th smallest
// (1-based) of histogram h[0..NB), and the rank left inside it
template <int NB, int NT>
CLSA_DEV void find_bin_asc(const uint32_t* h, uint32_t rank, uint32_t* tmp, uint32_t* out2) {
  constexpr int PER = NB / NT;
  const int tid = threadIdx.x;
  uint32_t v[PER], sum = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    v[i] = h[PER * tid + i];
    sum += v[i];
  }
  const uint32_t incl = block_incl_scan<NT>(sum, tmp);
  const uint32_t excl = incl - sum;
  if (excl < rank && rank <= incl) {
    uint32_t acc = excl;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (acc + v[i] >= rank) {
        out2[0] = (uint32_t)(PER * tid + i);
        out2[1] = rank - acc;
        break;
      }
      acc += v[i];
    }
  }
  __syncthreads();
}

template <int DS>
__global__ __launch_bounds__(kSplitThreads) void lv_split(SplitArgs a) {
  constexpr int NT = kSplitThreads;
  constexpr int kNs = kLvSampleFloats / DS < 256 ? kLvSampleFloats / DS : 256;
  __shared__ float xs[kNs][DS];  // centered samples
  __shared__ float mu[DS], v[DS], vn[DS];
  __shared__ float w[kNs];
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t tmp[NT / kWave];
  __shared__ uint32_t bc[4];
  __shared__ float nrm;

  const int i = blockIdx.x, bs = blockIdx.y;
  const int b = bs / a.S, s = bs % a.S;
  const int tid = threadIdx.x;
  const int64_t lo = ((int64_t)i * a.n) >> a.level;
  const int64_t hi = ((int64_t)(i + 1) * a.n) >> a.level;
  const int64_t mid = ((int64_t)(2 * i + 1) * a.n) >> (a.level + 1);
  const int64_t sz = hi - lo;
  uint32_t* keys = a.keys + (size_t)bs * a.n;
  int32_t* pout = a.pout + (size_t)bs * a.pout_stride + a.pout_off;

  // ---- sample: ns members at evenly spaced slots, centered ----
  const int ns = (int)(sz < kNs ? sz : kNs);
  for (int e = tid; e < ns * DS; e += NT) {
    const int t = e / DS, c = e % DS;
    const int32_t p = slot_pos(a, bs, lo + (int64_t)t * sz / ns);
    xs[t][c] = __uint_as_float((uint32_t)sub_row(a, b, s, p)[c] << 16);
  }
  __syncthreads();
  if (tid < DS) {
    float acc = 0.f;
    for (int t = 0; t < ns; ++t) acc += xs[t][tid];
    mu[tid] = acc / (float)ns;
    v[tid] = 1.0f + (float)tid / (float)DS;  // deterministic start, not symmetric
  }
  __syncthreads();
  for (int e = tid; e < ns * DS; e += NT) xs[e / DS][e % DS] -= mu[e % DS];
  __syncthreads();
  // ---- principal axis: power iteration on the sample's covariance ----
  for (int it = 0; it < kPowerIters; ++it) {
    for (int t = tid; t < ns; t += NT) {
      float acc = 0.f;
#pragma unroll 8
      for (int c = 0; c < DS; ++c) acc = fmaf(xs[t][c], v[c], acc);
      w[t] = acc;
    }
    __syncthreads();
    if (tid < DS) {
      float acc = 0.f;
      for (int t = 0; t < ns; ++t) acc = fmaf(w[t], xs[t][tid], acc);
      vn[tid] = acc;
    }
    __syncthreads();
    if (tid == 0) {
      float q = 0.f;
      for (int c = 0; c < DS; ++c) q = fmaf(vn[c], vn[c], q);
      nrm = q;
    }
    __syncthreads();
    if (tid < DS && nrm > 0.f) v[tid] = vn[tid] * rsqrtf(nrm);
    __syncthreads();
  }

  // ---- projections of every member (order-preserving keys) ----
  for (int64_t t = lo + tid; t < hi; t += NT) {
    const uint16_t* x = sub_row(a, b, s, slot_pos(a, bs, t));
    float acc = 0.f;
#pragma unroll
    for (int c0 = 0; c0 < DS; c0 += 8) {
      const u32x4_t q = *reinterpret_cast<const u32x4_t*>(x + c0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc = fmaf(bf16_lo(q[e]), v[c0 + 2 * e], acc);
        acc = fmaf(bf16_hi(q[e]), v[c0 + 2 * e + 1], acc);
      }
    }
    keys[t] = score_key(acc);
  }
  __syncthreads();

  // ---- the (mid - lo + 1)-th smallest key, exactly (three radix passes) ----
  uint32_t rank = (uint32_t)(mid - lo + 1);
  uint32_t prefix = 0, kstar = 0, left_eq = 0;
  const bool split = mid < hi;  // a node of one key has nothing to split
  if (split) {
#pragma unroll 1
    for (int pass = 0; pass < 3; ++pass) {
      const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
      const uint32_t width = pass == 2 ? 1023u : 2047u;
      const uint32_t pmask = pass == 0 ? 0u : (pass == 1 ? 0xFFE00000u : 0xFFFFFC00u);
      for (int e = tid; e < 2048; e += NT) hist[e] = 0u;
      __syncthreads();
      for (int64_t t = lo + tid; t < hi; t += NT) {
        const uint32_t k = keys[t];
        if ((k & pmask) == prefix) atomicAdd(&hist[(k >> shift) & width], 1u);
      }
      __syncthreads();
      find_bin_asc<2048, NT>(hist, rank, tmp, bc);
      prefix |= bc[0] << shift;
      rank = bc[1];
      __syncthreads();
    }
    kstar = prefix;
    left_eq = rank - 1;  // keys equal to kstar that still go left (slot order)
  }

  // ---- stable partition: keys below kstar, then the first left_eq equal
  //      ones, go left; the rest go right, both in slot order ----
  uint32_t nl = 0, nr = 0, neq = 0;
  for (int64_t t0 = lo; t0 < hi; t0 += NT) {
    const int64_t t = t0 + tid;
    const bool in = t < hi;
    const uint32_t k = in ? keys[t] : 0u;
    const bool eq = in && split && k == kstar;
    const uint32_t eq_before = neq + block_incl_scan<NT>(eq ? 1u : 0u, tmp) - (eq ? 1u : 0u);
    if (tid == NT - 1) bc[2] = eq_before + (eq ? 1u : 0u) - neq;
    const bool left = in && (!split || k < kstar || (eq && eq_before < left_eq));
    const uint32_t lb = block_incl_scan<NT>(left ? 1u : 0u, tmp) - (left ? 1u : 0u);
    if (tid == NT - 1) bc[3] = lb + (left ? 1u : 0u);
    __syncthreads();
    const uint32_t nleft = bc[3], neqc = bc[2];
    if (in) {
      const int32_t p = slot_pos(a, bs, t);
      if (left) pout[lo + nl + lb] = p;
      else pout[mid + nr + ((uint32_t)tid - lb)] = p;  // right ones before: tid - lb
    }
    nl += nleft;
    nr += (uint32_t)((hi - t0 < NT ? hi - t0 : NT)) - nleft;
    neq += neqc;
    __syncthreads();
  }
}

// a segment that fits one cluster: its slots in position order
__global__ __launch_bounds__(256) void lv_identity(int32_t* perm, int64_t n_max, int64_t a0,
                                                   int64_t n) {
  const int bs = blockIdx.y;
  for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < n; t += (int64_t)gridDim.x * 256)
    perm[(size_t)bs * n_max + a0 + t] = (int32_t)(a0 + t);
}

struct LeafArgs {
  const uint16_t* K;
  int64_t n_cap;
  int d, S, ds, h;
  int64_t a, n, n_max;
  int cbase, C_max;
  LvIndex ix;
};

// one wave per cluster: center (mean rounded to bf16), radius, cluster ids
template <int DS>
__global__ __launch_bounds__(64) void lv_leaves(LeafArgs a) {
  const int i = blockIdx.x, bs = blockIdx.y;
  const int b = bs / a.S, s = bs % a.S;
  const int lane = lane_id();
  const int64_t t0 = a.a + (((int64_t)i * a.n) >> a.h);
  const int64_t t1 = a.a + (((int64_t)(i + 1) * a.n) >> a.h);
  const int g = a.cbase + i;
  const int32_t* perm = a.ix.perm + (size_t)bs * a.n_max;
  const uint16_t* Kb = a.K + (size_t)b * a.n_cap * a.d + (size_t)s * a.ds;
  constexpr int kPer = DS > 64 ? DS / 64 : 1;
  float cf[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int c = lane + 64 * u;
    float acc = 0.f;
    if (c < DS)
      for (int64_t t = t0; t < t1; ++t)
        acc += __uint_as_float((uint32_t)Kb[(size_t)perm[t] * a.d + c] << 16);
    cf[u] = c < DS ? __uint_as_float((uint32_t)f32_to_bf16(acc / (float)(t1 - t0)) << 16) : 0.f;
    if (c < DS) a.ix.centers[(((size_t)bs * a.C_max) + g) * DS + c] = f32_to_bf16(cf[u]);
  }
  // radius from the stored (rounded) center; members spread over the lanes
  __shared__ float cs[DS];
#pragma unroll
  for (int u = 0; u < kPer; ++u)
    if (lane + 64 * u < DS) cs[lane + 64 * u] = cf[u];
  __builtin_amdgcn_wave_barrier();
  __syncthreads();
  float r2 = 0.f;
  for (int64_t t = t0 + lane; t < t1; t += 64) {
    const int32_t p = perm[t];
    const uint16_t* x = Kb + (size_t)p * a.d;
    float acc = 0.f;
    for (int c = 0; c < DS; ++c) {
      const float dx = __uint_as_float((uint32_t)x[c] << 16) - cs[c];
      acc = fmaf(dx, dx, acc);
    }
    r2 = fmaxf(r2, acc);
    if (a.S > 1) a.ix.cid[(size_t)bs * a.n_max + p] = (uint16_t)g;
  }
  r2 = wave_max(r2);
  if (lane == 0) {
    a.ix.radius[(size_t)bs * a.C_max + g] = sqrtf(r2) * (1.0f + 1.0f / 4096.0f);
    if (bs == 0) {
      a.ix.cl_begin[g] = (int32_t)t0;
      a.ix.cl_begin[g + 1] = (int32_t)t1;  // the next cluster overwrites it with the same value
    }
  }
}

// ================================================================= query
constexpr int kBufBlocks = 64;  // workgroups of the buffer scan per row

struct QueryArgs {
  const uint16_t* q;    // [B][d]
  const uint16_t* K;    // [B][n_cap][d]
  const int32_t* n_ctx;
  const float* tau;     // [B]
  int64_t n_cap, n_max;
  int B, d, S, ds, C_tot, C_max, nseg;
  int64_t idx_end;      // end of the last segment: positions >= idx_end are the buffer
  int seg_c[kLvMaxSegs + 1];  // first global cluster of each segment
  LvIndex ix;
  // workspace (nothing needs to be zero on entry: lv_bounds clears the hit
  // bitmap and the counters before any kernel reads them)
  float* ub;            // [B][S][C_tot] bound + margin
  float* ubmax;         // [B][S] largest bound per subspace (Query 1, S > 1)
  float* cut;           // [B][nseg][S] Query 2 cut per segment and subspace
  float* sorted;        // [B][S][C_tot] Query 2 bounds in descending order
  uint32_t* hit;        // [B][W] bitmap over positions
  uint32_t* ncl;        // [B][S][C_tot] keys a cluster's wave scored exactly
  uint32_t* nbuf;       // [B][kBufBlocks] keys of the buffer scored per workgroup
  int W;                // bitmap words per row
  int32_t* idx;
  int32_t* counts;
  int cap;
  uint32_t* checked_out;  // [B] or null
};

CLSA_DEV int64_t lv_visible(const QueryArgs& a, int b) {
  int64_t n = a.n_ctx ? (int64_t)a.n_ctx[b] : a.n_cap;
  return n < 0 ? 0 : (n > a.n_cap ? a.n_cap : n);
}

// Every cluster's bound in every subspace: <q_s, c> + rho |q_s| plus a
// margin far above the fp32 rounding of the dot product, the norm and the
// radius.  DS / 8 lanes share a cluster, 16 bytes of its center each.  The
// row's workgroups also clear its hit bitmap and counters.
template <int DS>
__global__ __launch_bounds__(256) void lv_bounds(QueryArgs a) {
  constexpr int LPC = DS / 8;       // lanes per cluster
  constexpr int CPB = 256 / LPC;    // clusters per workgroup
  const int b = blockIdx.y / a.S, s = blockIdx.y % a.S;
  const int tid = threadIdx.x;
  __shared__ float qn_s;
  // clear: the row's hit bitmap, its per-cluster counts and buffer counts
  {
    const int f = s * gridDim.x + blockIdx.x, nf = a.S * gridDim.x;
    for (int i = f * 256 + tid; i < a.W; i += nf * 256) a.hit[(size_t)b * a.W + i] = 0u;
    if (f == 0 && tid < kBufBlocks) a.nbuf[b * kBufBlocks + tid] = 0u;
  }
  const u32x4_t qv =
      *reinterpret_cast<const u32x4_t*>(a.q + (size_t)b * a.d + s * DS + (tid % LPC) * 8);
  if (tid < 64) {
    float acc = 0.f;
    for (int c = tid; c < DS; c += 64) {
      const float x = __uint_as_float((uint32_t)a.q[(size_t)b * a.d + s * DS + c] << 16);
      acc = fmaf(x, x, acc);
    }
    acc = wave_sum(acc);
    if (tid == 0) qn_s = sqrtf(acc) * (1.0f + 1.0f / 4096.0f);
  }
  __syncthreads();
  const float qn = qn_s;
  const int g = blockIdx.x * CPB + tid / LPC;
  const bool ok = g < a.C_tot;
  float dot = 0.f, mag = 0.f;
  if (ok) {
    const u32x4_t x = *reinterpret_cast<const u32x4_t*>(
        a.ix.centers + (((size_t)(b * a.S + s) * a.C_max) + g) * DS + (tid % LPC) * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float p0 = bf16_lo(qv[e]) * bf16_lo(x[e]);
      const float p1 = bf16_hi(qv[e]) * bf16_hi(x[e]);
      dot += p0 + p1;
      mag += fabsf(p0) + fabsf(p1);
    }
  }
#pragma unroll
  for (int m = LPC / 2; m >= 1; m >>= 1) {
    dot += __shfl_xor(dot, m);
    mag += __shfl_xor(mag, m);
  }
  if (ok && tid % LPC == 0) {
    const size_t o = ((size_t)b * a.S + s) * a.C_tot + g;
    const float rq = a.ix.radius[(size_t)(b * a.S + s) * a.C_max + g] * qn;
    a.ub[o] = dot + rq + 1e-4f * (mag + rq) + 1e-30f;
    a.ncl[o] = 0u;
  }
}

// Query 1 with S > 1: each subspace's largest bound (one workgroup per row
// and subspace, no atomics)
__global__ __launch_bounds__(256) void lv_max(QueryArgs a) {
  __shared__ float wm[4];
  const int bs = blockIdx.x;
  const float* u = a.ub + (size_t)bs * a.C_tot;
  float m = -INFINITY;
  for (int g = threadIdx.x; g < a.C_tot; g += 256) m = fmaxf(m, u[g]);
  m = wave_max(m);
  if (lane_id() == 0) wm[threadIdx.x / 64] = m;
  __syncthreads();
  if (threadIdx.x == 0) a.ubmax[bs] = fmaxf(fmaxf(wm[0], wm[1]), fmaxf(wm[2], wm[3]));
}

// Query 2: per (row, segment) the stop depth of the threshold algorithm and
// each subspace's cut, the bound at rank t* - 1 (+inf when t* = 0, -inf when
// the scan never stops).
constexpr int kTaMax = 8192;  // clusters of one segment
__global__ __launch_bounds__(1024) void lv_ta_depth(QueryArgs a) {
  __shared__ float srt[kTaMax];
  __shared__ int stop;
  const int b = blockIdx.y, k = blockIdx.x;
  const int tid = threadIdx.x;
  const int c0 = a.seg_c[k], C = a.seg_c[k + 1] - c0;
  int P = 1;
  while (P < C) P <<= 1;
  const float tau = a.tau[b];
  for (int s = 0; s < a.S; ++s) {
    const float* u = a.ub + ((size_t)b * a.S + s) * a.C_tot + c0;
    for (int e = tid; e < P; e += 1024) srt[e] = e < C ? u[e] : -INFINITY;
    __syncthreads();
    // bitonic sort, descending
    for (int kk = 2; kk <= P; kk <<= 1) {
      for (int j = kk >> 1; j > 0; j >>= 1) {
        for (int e = tid; e < P; e += 1024) {
          const int o = e ^ j;
          if (o > e) {
            const bool desc = (e & kk) == 0;
            const float x = srt[e], y = srt[o];
            if (desc ? (x < y) : (x > y)) {
              srt[e] = y;
              srt[o] = x;
            }
          }
        }
        __syncthreads();
      }
    }
    float* dst = a.sorted + ((size_t)b * a.S + s) * a.C_tot + c0;
    for (int e = tid; e < C; e += 1024) dst[e] = srt[e];
    __syncthreads();
  }
  if (tid == 0) stop = C;
  __syncthreads();
  // the bounds' sum falls with the depth: the first depth below tau
  for (int t = tid; t < C; t += 1024) {
    float sum = 0.f;
    for (int s = 0; s < a.S; ++s) sum += a.sorted[((size_t)b * a.S + s) * a.C_tot + c0 + t];
    if (sum < tau) atomicMin(&stop, t);
  }
  __syncthreads();
  const int ts = stop;
  if (tid < a.S) {
    const float cv = ts == 0 ? INFINITY
                             : (ts >= C ? -INFINITY
                                        : a.sorted[((size_t)b * a.S + tid) * a.C_tot + c0 + ts - 1]);
    a.cut[((size_t)b * a.nseg + k) * a.S + tid] = cv;
  }
}

CLSA_DEV int seg_of(const QueryArgs& a, int g) {
  int k = 0;
  while (k + 1 < a.nseg && g >= a.seg_c[k + 1]) ++k;
  return k;
}

CLSA_DEV void mark_hit(const QueryArgs& a, int b, int32_t p) {
  atomicOr(&a.hit[(size_t)b * a.W + (p >> 5)], 1u << (p & 31));
}

// exact score of one key row: the LPK lanes of a key group hold 16 bytes
// each; the sum is complete in every lane of the group
template <int LPK>
CLSA_DEV float row_dot(const u32x4_t& x, const u32x4_t& qv) {
  float acc = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    acc = fmaf(bf16_lo(qv[e]), bf16_lo(x[e]), acc);
    acc = fmaf(bf16_hi(qv[e]), bf16_hi(x[e]), acc);
  }
#pragma unroll
  for (int m = LPK / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
  return acc;
}

// MODE 1: Query 1 (one wave per cluster of subspace 0); MODE 2: Query 2
// (one wave per cluster and subspace).  D: full key width.
// A passing cluster's members are taken 64 at a time: one slot per lane,
// the member's candidacy decided in its own lane, then every key row of the
// 64 requested together (D/8 lanes per row), so a cluster costs a few
// memory round trips rather than one per key group.  In Query 2 a key
// whose cluster is seen in several subspaces is scored from the lowest of
// them only.  Each wave writes how many keys it scored; nothing is counted
// with atomics on one address (device-scope atomics to one word serialize).
template <int D, int MODE>
__global__ __launch_bounds__(64 * kScanWaves) void lv_scan(QueryArgs a) {
  constexpr int LPK = D / 8;
  constexpr int KPW = 64 / LPK;  // key rows per wave load
  constexpr int NL = 64 / KPW;   // loads covering 64 members
  const int lane = lane_id(), w = threadIdx.x / kWave;
  const int g = blockIdx.x * kScanWaves + w;
  const int b = MODE == 1 ? blockIdx.y : blockIdx.y / a.S;
  const int s = MODE == 1 ? 0 : blockIdx.y % a.S;
  if (g >= a.C_tot) return;
  const float tau = a.tau[b];
  const int64_t n_vis = lv_visible(a, b);
  const float u = a.ub[((size_t)b * a.S + s) * a.C_tot + g];
  const int k = seg_of(a, g);
  const float* cut = a.cut + ((size_t)b * a.nseg + k) * a.S;
  float thr;
  if (MODE == 1) {  // tau minus the other subspaces' largest bounds
    float others = 0.f;
    for (int s2 = 1; s2 < a.S; ++s2) others += a.ubmax[b * a.S + s2];
    thr = tau - others;
  } else {
    thr = cut[s];
  }
  if (!(u >= thr)) return;  // the ball misses the half-space (wave-uniform)
  const u32x4_t qv = *reinterpret_cast<const u32x4_t*>(a.q + (size_t)b * D + (lane % LPK) * 8);
  const int32_t* perm = a.ix.perm + (size_t)(b * a.S + s) * a.n_max;
  const int t0 = a.ix.cl_begin[g], t1 = a.ix.cl_begin[g + 1];
  uint32_t nchk = 0;
  for (int c0 = t0; c0 < t1; c0 += 64) {
    // this lane's member: its position and whether it is scored here
    const int t = c0 + lane;
    const int32_t p = t < t1 ? perm[t] : -1;
    bool cand = p >= 0 && p < n_vis;
    if (a.S > 1 && cand) {
      if (MODE == 1) {
        // the member's clusters in the other subspaces must pass too
        float tot = 0.f;
        for (int s2 = 0; s2 < a.S; ++s2) tot += a.ubmax[b * a.S + s2];
        for (int s2 = 1; s2 < a.S; ++s2) {
          const int g2 = a.ix.cid[(size_t)(b * a.S + s2) * a.n_max + p];
          const float thr2 = tau - (tot - a.ubmax[b * a.S + s2]);
          cand = cand && a.ub[((size_t)b * a.S + s2) * a.C_tot + g2] >= thr2;
        }
      } else {
        // seen from a lower subspace: scored there
        for (int s2 = 0; s2 < s; ++s2) {
          const int g2 = a.ix.cid[(size_t)(b * a.S + s2) * a.n_max + p];
          cand = cand && !(a.ub[((size_t)b * a.S + s2) * a.C_tot + g2] >= cut[s2]);
        }
      }
    }
    const uint64_t cm = __ballot(cand);
    if (cm == 0ull) continue;
    nchk += (uint32_t)__popcll(cm);
    // the key rows of all 64 members, requested together
    u32x4_t x[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int src = i * KPW + lane / LPK;  // member served by this lane group
      const int32_t pp = __shfl(p, src);
      x[i] = u32x4_t{0u, 0u, 0u, 0u};
      if ((cm >> src) & 1ull)
        x[i] = *reinterpret_cast<const u32x4_t*>(a.K + ((size_t)b * a.n_cap + pp) * D +
                                                 (lane % LPK) * 8);
    }
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int src = i * KPW + lane / LPK;
      const float sc = row_dot<LPK>(x[i], qv);
      const int32_t pp = __shfl(p, src);
      if ((lane % LPK) == 0 && ((cm >> src) & 1ull) && sc >= tau) mark_hit(a, b, pp);
    }
  }
  if (lane == 0) a.ncl[((size_t)b * a.S + s) * a.C_tot + g] = nchk;
}

// the buffer: positions idx_end .. n_vis - 1, checked exactly
template <int D>
__global__ __launch_bounds__(256) void lv_buffer(QueryArgs a) {
  constexpr int LPK = D / 8;
  constexpr int KPW = 64 / LPK;
  __shared__ uint32_t wn[4];
  const int b = blockIdx.y;
  const int lane = lane_id(), w = threadIdx.x / kWave;
  const int64_t n_vis = lv_visible(a, b);
  const float tau = a.tau[b];
  const u32x4_t qv = *reinterpret_cast<const u32x4_t*>(a.q + (size_t)b * D + (lane % LPK) * 8);
  uint32_t nchk = 0;
  for (int64_t tb = a.idx_end + ((int64_t)blockIdx.x * 4 + w) * KPW; tb < n_vis;
       tb += (int64_t)gridDim.x * 4 * KPW) {
    const int64_t p = tb + lane / LPK;
    const bool v = p < n_vis;
    u32x4_t x = {0u, 0u, 0u, 0u};
    if (v)
      x = *reinterpret_cast<const u32x4_t*>(a.K + ((size_t)b * a.n_cap + p) * D + (lane % LPK) * 8);
    const float sc = row_dot<LPK>(x, qv);
    if (v && (lane % LPK) == 0) {
      ++nchk;
      if (sc >= tau) mark_hit(a, b, (int32_t)p);
    }
  }
  nchk = wave_sum_u32(nchk);
  if (lane == 0) wn[w] = nchk;
  __syncthreads();
  if (threadIdx.x == 0) a.nbuf[b * kBufBlocks + blockIdx.x] = wn[0] + wn[1] + wn[2] + wn[3];
}

// positions of the row's bitmap in ascending order, the true count, and the
// number of keys the query scored
__global__ __launch_bounds__(1024) void lv_compact(QueryArgs a) {
  __shared__ uint32_t tmp[16];
  __shared__ uint32_t total;
  const int b = blockIdx.x, tid = threadIdx.x;
  const int64_t n_vis = lv_visible(a, b);
  const int W = (int)ceil_div64(n_vis, 32);
  const int per = (W + 1023) / 1024;
  const uint32_t* hb = a.hit + (size_t)b * a.W;
  const int w0 = tid * per;
  uint32_t mine = 0;
  for (int i = w0; i < w0 + per && i < W; ++i) mine += __popc(hb[i]);
  const uint32_t incl = block_incl_scan<1024>(mine, tmp);
  uint32_t run = incl - mine;
  int32_t* out = a.idx + (size_t)b * a.cap;
  for (int i = w0; i < w0 + per && i < W; ++i) {
    uint32_t x = hb[i];
    while (x) {
      const int bit = __builtin_ctz(x);
      x &= x - 1u;
      if (run < (uint32_t)a.cap) out[run] = i * 32 + bit;
      ++run;
    }
  }
  if (tid == 1023) {
    total = incl;
    a.counts[b] = (int32_t)incl;
  }
  __syncthreads();
  for (int64_t i = (int64_t)total + tid; i < a.cap; i += 1024) out[i] = -1;
  if (a.checked_out) {
    uint32_t c = 0;
    const uint32_t* n = a.ncl + (size_t)b * a.S * a.C_tot;
    for (int i = tid; i < a.S * a.C_tot; i += 1024) c += n[i];
    if (tid < kBufBlocks) c += a.nbuf[b * kBufBlocks + tid];
    c = block_incl_scan<1024>(c, tmp);
    if (tid == 1023) a.checked_out[b] = c;
  }
}

bool lv_shape_ok(int B, int d, int S, int r) {
  if (B < 1 || B > 65535 / 4) return false;
  if (d != 32 && d != 64 && d != 128) return false;
  if (S != 1 && S != 2 && S != 4) return false;
  const int ds = d / S;
  if (ds < 8 || ds % 8 != 0) return false;
  return r >= 8 && r <= 256;
}

// the segment table: bounds[0] = 0 < bounds[1] < ... <= n_max; cluster
// bases per segment
bool lv_segments(int nseg, const int64_t* bounds, int64_t n_max, int r, int C_max,
                 int* seg_c) {
  if (nseg < 1 || nseg > kLvMaxSegs || !bounds || bounds[0] != 0) return false;
  int c = 0;
  for (int k = 0; k < nseg; ++k) {
    if (bounds[k + 1] <= bounds[k] || bounds[k + 1] > n_max) return false;
    seg_c[k] = c;
    const int h = tree_levels(bounds[k + 1] - bounds[k], r);
    if (h > 13) return false;  // more than 8192 clusters in one segment
    c += 1 << h;
  }
  seg_c[nseg] = c;
  return c <= C_max && c <= 65535;
}

template <int DS>
void launch_split(const SplitArgs& sa, int nodes, int BS, hipStream_t s) {
  hipLaunchKernelGGL(lv_split<DS>, dim3((unsigned)nodes, (unsigned)BS), dim3(kSplitThreads), 0,
                     s, sa);
}
template <int DS>
void launch_leaves(const LeafArgs& la, int C, int BS, hipStream_t s) {
  hipLaunchKernelGGL(lv_leaves<DS>, dim3((unsigned)C, (unsigned)BS), dim3(64), 0, s, la);
}
#define CLSA_DS_SWITCH(ds, F, ...)         \
  switch (ds) {                            \
    case 8: F<8>(__VA_ARGS__); break;      \
    case 16: F<16>(__VA_ARGS__); break;    \
    case 32: F<32>(__VA_ARGS__); break;    \
    case 64: F<64>(__VA_ARGS__); break;    \
    default: F<128>(__VA_ARGS__); break;   \
  }

struct QueryLayout {
  int W;
  size_t o_ub, o_ubmax, o_cut, o_sorted, o_hit, o_ncl, o_nbuf, total;
};
QueryLayout lv_query_layout(int B, int64_t n_cap, int S, int C_tot, int nseg) {
  QueryLayout Q{};
  Q.W = (int)ceil_div64(n_cap, 32);
  size_t o = 0;
  Q.o_ub = o; o = align_up(o + (size_t)B * S * C_tot * 4, 256);
  Q.o_ubmax = o; o = align_up(o + (size_t)B * S * 4, 256);
  Q.o_cut = o; o = align_up(o + (size_t)B * nseg * S * 4, 256);
  Q.o_sorted = o; o = align_up(o + (size_t)B * S * C_tot * 4, 256);
  Q.o_hit = o; o = align_up(o + (size_t)B * Q.W * 4, 256);
  Q.o_ncl = o; o = align_up(o + (size_t)B * S * C_tot * 4, 256);
  Q.o_nbuf = o; o = align_up(o + (size_t)B * kBufBlocks * 4, 256);
  Q.total = o;
  return Q;
}

template <int DS>
void launch_bounds_ds(const QueryArgs& qa, hipStream_t s) {
  constexpr int CPB = 256 / (DS / 8);
  hipLaunchKernelGGL(lv_bounds<DS>, dim3((unsigned)ceil_div64(qa.C_tot, CPB), (unsigned)(qa.B * qa.S)),
                     dim3(256), 0, s, qa);
}

template <int D>
void launch_query(const QueryArgs& qa, int mode, hipStream_t s) {
  CLSA_DS_SWITCH(qa.ds, launch_bounds_ds, qa, s);
  const unsigned gw = (unsigned)ceil_div64(qa.C_tot, kScanWaves);
  if (mode == 1) {
    if (qa.S > 1)
      hipLaunchKernelGGL(lv_max, dim3((unsigned)(qa.B * qa.S)), dim3(256), 0, s, qa);
    hipLaunchKernelGGL((lv_scan<D, 1>), dim3(gw, (unsigned)qa.B), dim3(64 * kScanWaves), 0, s,
                       qa);
  } else {
    hipLaunchKernelGGL(lv_ta_depth, dim3((unsigned)qa.nseg, (unsigned)qa.B), dim3(1024), 0, s,
                       qa);
    hipLaunchKernelGGL((lv_scan<D, 2>), dim3(gw, (unsigned)(qa.B * qa.S)),
                       dim3(64 * kScanWaves), 0, s, qa);
  }
  if (qa.idx_end < qa.n_cap)  // some sequence may hold keys past the index
    hipLaunchKernelGGL(lv_buffer<D>, dim3((unsigned)kBufBlocks, (unsigned)qa.B), dim3(256), 0,
                       s, qa);
  hipLaunchKernelGGL(lv_compact, dim3((unsigned)qa.B), dim3(1024), 0, s, qa);
}

}  // namespace
}  // namespace clsa

using namespace clsa;

extern "C" size_t clsa_louver_index_bytes(int B, int d, int64_t n_max, int S, int r) {
  if (!lv_shape_ok(B, d, S, r) || n_max < 1 || n_max > (int64_t)1 << 24) return 0;
  return lv_layout(B, d, n_max, S, r).total;
}

extern "C" size_t clsa_louver_build_workspace_size(int B, int d, int64_t n_max, int S, int r) {
  if (!lv_shape_ok(B, d, S, r) || n_max < 1 || n_max > (int64_t)1 << 24) return 0;
  (void)d;
  // projection keys and two slot -> position buffers, per (sequence, subspace)
  return align_up((size_t)B * S * n_max * 4, 256) * 3;
}

extern "C" int clsa_louver_build(const void* K_idx, int B, int d, int64_t n_cap, clsa_dtype dt,
                                 int S, int r, int64_t n_max, int nseg, const int64_t* seg_bounds,
                                 void* index, size_t index_bytes, void* ws, size_t ws_bytes,
                                 void* stream) {
  if (dt != CLSA_BF16) return CLSA_ERR_UNSUPPORTED_DTYPE;
  if (!K_idx || !index || !lv_shape_ok(B, d, S, r) || n_max < 1 || n_max > (int64_t)1 << 24 ||
      n_cap < 1 || n_cap > 0x7fffffff)
    return CLSA_ERR_INVALID;
  const LvLayout L = lv_layout(B, d, n_max, S, r);
  int seg_c[kLvMaxSegs + 1];
  if (!lv_segments(nseg, seg_bounds, n_max, r, L.C_max, seg_c)) return CLSA_ERR_INVALID;
  const int64_t a0 = seg_bounds[nseg - 1], a1 = seg_bounds[nseg];
  if (a1 > n_cap) return CLSA_ERR_INVALID;
  if (index_bytes < L.total) return CLSA_ERR_INVALID;
  const size_t need = clsa_louver_build_workspace_size(B, d, n_max, S, r);
  if (!ws || ws_bytes < need) return CLSA_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const LvIndex ix = lv_index(index, L);
  const int ds = d / S, BS = B * S;
  const int64_t n = a1 - a0;
  const int h = tree_levels(n, r);
  const size_t part = align_up((size_t)BS * n_max * 4, 256);
  char* w = static_cast<char*>(ws);
  uint32_t* keys = reinterpret_cast<uint32_t*>(w);
  int32_t* buf[2] = {reinterpret_cast<int32_t*>(w + part), reinterpret_cast<int32_t*>(w + 2 * part)};

  SplitArgs sa{};
  sa.K = static_cast<const uint16_t*>(K_idx);
  sa.n_cap = n_cap;
  sa.d = d;
  sa.S = S;
  sa.ds = ds;
  sa.a = a0;
  sa.n = n;
  sa.keys = keys;
  if (h == 0)
    hipLaunchKernelGGL(lv_identity, dim3((unsigned)ceil_div64(n, 256), (unsigned)BS), dim3(256), 0,
                       s, ix.perm, n_max, a0, n);
  for (int lv = 0; lv < h; ++lv) {
    sa.level = lv;
    sa.pin = lv == 0 ? nullptr : buf[(lv - 1) & 1];
    const bool last = lv == h - 1;
    sa.pout = last ? ix.perm : buf[lv & 1];
    sa.pout_stride = last ? n_max : n;
    sa.pout_off = last ? a0 : 0;
    CLSA_DS_SWITCH(ds, launch_split, sa, 1 << lv, BS, s);
  }
  LeafArgs la{};
  la.K = sa.K;
  la.n_cap = n_cap;
  la.d = d;
  la.S = S;
  la.ds = ds;
  la.h = h;
  la.a = a0;
  la.n = n;
  la.n_max = n_max;
  la.cbase = seg_c[nseg - 1];
  la.C_max = L.C_max;
  la.ix = ix;
  CLSA_DS_SWITCH(ds, launch_leaves, la, 1 << h, BS, s);
  return hipGetLastError() == hipSuccess ? CLSA_OK : CLSA_ERR_HIP;
}

extern "C" size_t clsa_louver_query_workspace_size(int B, int d, int64_t n_cap, int S, int r,
                                                   int64_t n_max, int nseg,
                                                   const int64_t* seg_bounds) {
  if (!lv_shape_ok(B, d, S, r) || n_max < 1 || n_max > (int64_t)1 << 24 || n_cap < 1 ||
      n_cap > 0x7fffffff)
    return 0;
  int seg_c[kLvMaxSegs + 1];
  if (!lv_segments(nseg, seg_bounds, n_max, r, lv_layout(B, d, n_max, S, r).C_max, seg_c))
    return 0;
  return lv_query_layout(B, n_cap, S, seg_c[nseg], nseg).total;
}

extern "C" int clsa_louver_query(const void* q_idx, const void* K_idx, int B, int d,
                                 int64_t n_cap, const int32_t* n_ctx, const float* tau,
                                 clsa_dtype dt, int S, int r, int64_t n_max, int nseg,
                                 const int64_t* seg_bounds, const void* index, int mode,
                                 int32_t* idx, int32_t* counts, int cap, uint32_t* checked,
                                 void* ws, size_t ws_bytes, void* stream) {
  if (dt != CLSA_BF16) return CLSA_ERR_UNSUPPORTED_DTYPE;
  if (!q_idx || !K_idx || !tau || !index || !idx || !counts || cap < 1) return CLSA_ERR_INVALID;
  if (mode != 1 && mode != 2) return CLSA_ERR_INVALID;
  if (!lv_shape_ok(B, d, S, r) || n_max < 1 || n_max > (int64_t)1 << 24 || n_cap < 1 ||
      n_cap > 0x7fffffff)
    return CLSA_ERR_INVALID;
  const LvLayout L = lv_layout(B, d, n_max, S, r);
  QueryArgs qa{};
  if (!lv_segments(nseg, seg_bounds, n_max, r, L.C_max, qa.seg_c)) return CLSA_ERR_INVALID;
  if (seg_bounds[nseg] > n_cap) return CLSA_ERR_INVALID;
  const int C_tot = qa.seg_c[nseg];
  const QueryLayout Q = lv_query_layout(B, n_cap, S, C_tot, nseg);
  if (!ws || ws_bytes < Q.total) return CLSA_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  qa.q = static_cast<const uint16_t*>(q_idx);
  qa.K = static_cast<const uint16_t*>(K_idx);
  qa.n_ctx = n_ctx;
  qa.tau = tau;
  qa.n_cap = n_cap;
  qa.n_max = n_max;
  qa.B = B;
  qa.d = d;
  qa.S = S;
  qa.ds = d / S;
  qa.C_tot = C_tot;
  qa.C_max = L.C_max;
  qa.nseg = nseg;
  qa.idx_end = seg_bounds[nseg];
  qa.ix = lv_index(const_cast<void*>(index), L);
  qa.ub = reinterpret_cast<float*>(w + Q.o_ub);
  qa.ubmax = reinterpret_cast<float*>(w + Q.o_ubmax);
  qa.cut = reinterpret_cast<float*>(w + Q.o_cut);
  qa.sorted = reinterpret_cast<float*>(w + Q.o_sorted);
  qa.hit = reinterpret_cast<uint32_t*>(w + Q.o_hit);
  qa.ncl = reinterpret_cast<uint32_t*>(w + Q.o_ncl);
  qa.nbuf = reinterpret_cast<uint32_t*>(w + Q.o_nbuf);
  qa.W = Q.W;
  qa.idx = idx;
  qa.counts = counts;
  qa.cap = cap;
  qa.checked_out = checked;
  if (d == 32) launch_query<32>(qa, mode, s);
  else if (d == 64) launch_query<64>(qa, mode, s);
  else launch_query<128>(qa, mode, s);
  return hipGetLastError() == hipSuccess ? CLSA_OK : CLSA_ERR_HIP;
}

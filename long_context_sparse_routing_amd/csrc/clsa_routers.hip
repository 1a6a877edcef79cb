// Centroid table router: decode routing through a table built at prefill.
//
// Method: CSAttention summary (news.neo-ai.one, the article on CSAttention
// and STACK) -- a long context's queries are not spread evenly, so clustering
// them into centroids predicts which keys matter; the heavy work is done at
// prefill, where a fixed-size query-centroid lookup table is built per
// request, and decoding consults the table instead of scanning the whole
// context, with the scores still accumulated on the GPU.
//
// Build (per sequence: M prefill routing queries, C centroids):
//   km_init     centroid c starts at query floor(c M / C)
//   km_assign   each query's nearest centroid (squared Euclidean distance,
//               fp32, ties to the lower centroid)
//   km_update   each centroid the mean of its queries, summed in a fixed
//               order (an empty cluster keeps its centroid)
//   km_store    the centroids rounded to bf16 -- the table's keys
//   then clsa_route with the C centroids as query rows and k = T writes the
//   table: each centroid's T highest-scoring keys, ascending.
// Lookup (one query row per sequence):
//   csa_probe   the query's scores against the C centroids; its P best
//   csa_score   the candidates -- the P table rows and the positions past the
//               table (keys appended since it was built) -- scored exactly,
//               one wave per 64 candidates, D/8 lanes per key row
//   csa_select  per row: duplicates (a key in two probed rows) dropped, then
//               the exact top-k of the candidates in position order
#include "clsa_common.h"
#include "clsa_select.h"

namespace clsa {
namespace {

constexpr int kCsaMaxC = 1024;     // centroids per sequence
constexpr int kCsaMaxP = 16;       // centroids probed per query
constexpr int kCsaCap = 8192;      // candidates per row (table rows + buffer)
constexpr int kCsaPerT = kCsaCap / kSelNT;

// ---------------------------------------------------------------- k-means
struct KmArgs {
  const uint16_t* q;  // [B][M][d] bf16 prefill routing queries
  int B, M, d, C;
  float* mu;          // [B][C][d]
  int32_t* assign;    // [B][M]
  uint16_t* cent;     // [B][C][d] bf16 out
};

__global__ __launch_bounds__(128) void km_init(KmArgs a) {
  const int c = blockIdx.x, b = blockIdx.y;
  const int m = (int)((int64_t)c * a.M / a.C);
  for (int e = threadIdx.x; e < a.d; e += 128)
    a.mu[((size_t)b * a.C + c) * a.d + e] =
        __uint_as_float((uint32_t)a.q[((size_t)b * a.M + m) * a.d + e] << 16);
}

// one thread per query; the centroids of the sequence in LDS
template <int D>
__global__ __launch_bounds__(256) void km_assign(KmArgs a) {
  extern __shared__ float smu[];  // [C][D]
  const int b = blockIdx.y;
  for (int i = threadIdx.x; i < a.C * D; i += 256) smu[i] = a.mu[(size_t)b * a.C * D + i];
  __syncthreads();
  const int m = blockIdx.x * 256 + threadIdx.x;
  if (m >= a.M) return;
  uint32_t qw[D / 2];  // the query as bf16 pairs
  const uint32_t* qr = reinterpret_cast<const uint32_t*>(a.q + ((size_t)b * a.M + m) * D);
#pragma unroll
  for (int e = 0; e < D / 2; ++e) qw[e] = qr[e];
  float best = INFINITY;
  int bc = 0;
  for (int c = 0; c < a.C; ++c) {
    const float* mc = smu + c * D;
    float d2 = 0.f;
#pragma unroll
    for (int e = 0; e < D / 2; ++e) {
      const float x0 = bf16_lo(qw[e]) - mc[2 * e];
      const float x1 = bf16_hi(qw[e]) - mc[2 * e + 1];
      d2 = fmaf(x0, x0, d2);
      d2 = fmaf(x1, x1, d2);
    }
    if (d2 < best) {  // strict: ties keep the lower centroid
      best = d2;
      bc = c;
    }
  }
  a.assign[(size_t)b * a.M + m] = bc;
}

// one workgroup per centroid: wave w gathers the members among queries
// w M/4 .. (w+1) M/4 - 1 in ascending order (ballots of 64) and sums their
// rows, lane e holding dims e and e + 64; the four waves' sums are added in
// wave order, so the result does not depend on timing
template <int D>
__global__ __launch_bounds__(256) void km_update(KmArgs a) {
  constexpr int kPer = D > 64 ? 2 : 1;
  __shared__ float part[4][D];
  __shared__ uint32_t pcnt[4];
  const int c = blockIdx.x, b = blockIdx.y;
  const int lane = lane_id(), w = threadIdx.x / kWave;
  const int m0 = (int)((int64_t)w * a.M / 4), m1 = (int)((int64_t)(w + 1) * a.M / 4);
  float acc[kPer] = {};
  uint32_t n = 0;
  const int32_t* as = a.assign + (size_t)b * a.M;
  for (int mb = m0; mb < m1; mb += kWave) {
    const int m = mb + lane;
    uint64_t mask = __ballot(m < m1 && as[m] == c);
    n += (uint32_t)__popcll(mask);
    while (mask) {
      const int i = __builtin_ctzll(mask);
      mask &= mask - 1ull;
      const uint16_t* row = a.q + ((size_t)b * a.M + mb + i) * D;
#pragma unroll
      for (int u = 0; u < kPer; ++u)
        if (lane + 64 * u < D) acc[u] += __uint_as_float((uint32_t)row[lane + 64 * u] << 16);
    }
  }
#pragma unroll
  for (int u = 0; u < kPer; ++u)
    if (lane + 64 * u < D) part[w][lane + 64 * u] = acc[u];
  if (lane == 0) pcnt[w] = n;
  __syncthreads();
  const uint32_t tot = pcnt[0] + pcnt[1] + pcnt[2] + pcnt[3];
  if (tot == 0u) return;  // an empty cluster keeps its centroid
  for (int e = threadIdx.x; e < D; e += 256)
    a.mu[((size_t)b * a.C + c) * D + e] =
        (((part[0][e] + part[1][e]) + part[2][e]) + part[3][e]) / (float)tot;
}

__global__ __launch_bounds__(256) void km_store(KmArgs a) {
  const size_t n = (size_t)a.B * a.C * a.d;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256)
    a.cent[i] = f32_to_bf16(a.mu[i]);
}

// ----------------------------------------------------------------- lookup
struct CsaArgs {
  const uint16_t* q;      // [B][d]
  const uint16_t* K;      // [B][n_cap][d]
  const int32_t* n_ctx;
  const uint16_t* cent;   // [B][C][d] bf16
  const int32_t* table;   // [B][C][T]
  int64_t n_cap, n_table;
  int B, d, C, T, P, k, cap;
  int nbuf;               // buffer slots per row: n_cap - n_table
  int32_t* probe;         // [B][P] probed centroids (workspace)
  uint64_t* cand;         // [B][kCsaCap] (score bits << 32) | position; position ~0 = none
  int32_t* idx;
  int32_t* counts;
};

CLSA_DEV int64_t csa_visible(const CsaArgs& a, int b) {
  int64_t n = a.n_ctx ? (int64_t)a.n_ctx[b] : a.n_cap;
  return n < 0 ? 0 : (n > a.n_cap ? a.n_cap : n);
}

// the query's P best centroids (ties to the lower centroid)
template <int D>
__global__ __launch_bounds__(256) void csa_probe(CsaArgs a) {
  __shared__ float cs[kCsaMaxC];
  __shared__ float qs[D];
  __shared__ float wv[4];
  __shared__ int wi[4];
  const int b = blockIdx.x, tid = threadIdx.x;
  if (tid < D) qs[tid] = __uint_as_float((uint32_t)a.q[(size_t)b * D + tid] << 16);
  __syncthreads();
  for (int c = tid; c < a.C; c += 256) {
    const uint32_t* cr = reinterpret_cast<const uint32_t*>(a.cent + ((size_t)b * a.C + c) * D);
    float s = 0.f;
#pragma unroll 8
    for (int e = 0; e < D / 2; ++e) {
      const uint32_t x = cr[e];
      s = fmaf(qs[2 * e], bf16_lo(x), s);
      s = fmaf(qs[2 * e + 1], bf16_hi(x), s);
    }
    cs[c] = s;
  }
  __syncthreads();
  for (int p = 0; p < a.P; ++p) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    for (int c = tid; c < a.C; c += 256)
      if (cs[c] > bv || (cs[c] == bv && c < bi)) bv = cs[c], bi = c;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      const float ov = __shfl_xor(bv, m);
      const int oi = __shfl_xor(bi, m);
      if (ov > bv || (ov == bv && oi < bi)) bv = ov, bi = oi;
    }
    if (lane_id() == 0) wv[tid / 64] = bv, wi[tid / 64] = bi;
    __syncthreads();
    if (tid == 0) {
      float v = wv[0];
      int i = wi[0];
      for (int w = 1; w < 4; ++w)
        if (wv[w] > v || (wv[w] == v && wi[w] < i)) v = wv[w], i = wi[w];
      a.probe[b * a.P + p] = i;
      cs[i] = -INFINITY;  // taken
    }
    __syncthreads();
  }
}

// exact scores of the candidates: slot s < P T is entry s % T of the table
// row of probe s / T; slot P T + i is buffer position n_table + i
template <int D>
__global__ __launch_bounds__(256) void csa_score(CsaArgs a) {
  constexpr int LPK = D / 8;
  constexpr int KPW = 64 / LPK;
  constexpr int NL = 64 / KPW;
  const int b = blockIdx.y;
  const int lane = lane_id(), w = threadIdx.x / kWave;
  const int s0 = (blockIdx.x * 4 + w) * 64;
  const int nslot = a.P * a.T + a.nbuf;
  if (s0 >= nslot) return;
  const int64_t n_vis = csa_visible(a, b);
  const int sl = s0 + lane;
  int32_t p = -1;
  if (sl < a.P * a.T) {
    const int c = a.probe[b * a.P + sl / a.T];
    p = a.table[((size_t)b * a.C + c) * a.T + sl % a.T];
  } else if (sl < nslot) {
    p = (int32_t)(a.n_table + (sl - a.P * a.T));
  }
  const bool valid = p >= 0 && p < n_vis;
  const uint64_t vm = __ballot(valid);
  const u32x4_t qv = *reinterpret_cast<const u32x4_t*>(a.q + (size_t)b * D + (lane % LPK) * 8);
  u32x4_t x[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int src = i * KPW + lane / LPK;
    const int32_t pp = __shfl(p, src);
    x[i] = u32x4_t{0u, 0u, 0u, 0u};
    if ((vm >> src) & 1ull)
      x[i] = *reinterpret_cast<const u32x4_t*>(a.K + ((size_t)b * a.n_cap + pp) * D + (lane % LPK) * 8);
  }
  uint64_t* out = a.cand + (size_t)b * kCsaCap;
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int src = i * KPW + lane / LPK;
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc = fmaf(bf16_lo(qv[e]), bf16_lo(x[i][e]), acc);
      acc = fmaf(bf16_hi(qv[e]), bf16_hi(x[i][e]), acc);
    }
#pragma unroll
    for (int m = LPK / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
    const int32_t pp = __shfl(p, src);
    if ((lane % LPK) == 0 && s0 + src < nslot)
      out[s0 + src] = ((vm >> src) & 1ull)
                          ? (((uint64_t)__float_as_uint(acc) << 32) | (uint32_t)pp)
                          : ~0ull;
  }
}

// per row: drop duplicate candidates, then the exact top-k in order
__global__ __launch_bounds__(kSelNT) void csa_select(CsaArgs a) {
  extern __shared__ u32x4_t bitmap4[];  // positions bitmap + word prefixes
  uint32_t* bitmap = reinterpret_cast<uint32_t*>(bitmap4);
  __shared__ SelScratch S;
  __shared__ uint32_t tot;
  const int b = blockIdx.x, tid = threadIdx.x;
  const int wpt = (int)((ceil_div64(ceil_div64(a.n_cap, 32), kSelNT) + 3) / 4 * 4);
  const int w0 = tid * wpt;
  for (int i = w0; i < w0 + wpt; i += 4) bitmap4[i / 4] = u32x4_t{0u, 0u, 0u, 0u};
  if (tid == 0) tot = 0u;
  const int nslot = a.P * a.T + a.nbuf;
  const uint64_t* cr = a.cand + (size_t)b * kCsaCap;
  uint64_t e[kCsaPerT];
#pragma unroll
  for (int u = 0; u < kCsaPerT; ++u) {
    const int sl = u * kSelNT + tid;
    e[u] = sl < nslot ? cr[sl] : ~0ull;
  }
  __syncthreads();
  // keep the first copy of each position (copies are bit-identical: the
  // same key scored the same way); dropped and empty slots get key 0, below
  // every real score's key, and position 0
  uint32_t key[kCsaPerT], pos[kCsaPerT], mine = 0;
#pragma unroll
  for (int u = 0; u < kCsaPerT; ++u) {
    bool keep = e[u] != ~0ull;
    const uint32_t p = (uint32_t)e[u];
    if (keep) {
      const uint32_t bit = 1u << (p & 31);
      keep = (atomicOr(&bitmap[p >> 5], bit) & bit) == 0u;
    }
    key[u] = keep ? score_key(__uint_as_float((uint32_t)(e[u] >> 32))) : 0u;
    pos[u] = keep ? p : 0u;
    mine += keep ? 1u : 0u;
  }
  atomicAdd(&tot, mine);
  __syncthreads();
  const uint32_t n_c = tot;
  const uint32_t k_eff = (uint32_t)a.k < n_c ? (uint32_t)a.k : n_c;
  int32_t* out = a.idx + (size_t)b * a.cap;
  if (tid == 0) a.counts[b] = (int32_t)k_eff;
  for (int64_t i = k_eff + tid; i < a.cap; i += kSelNT) out[i] = -1;
  if (k_eff == 0u) return;
  // the bitmap held the candidates; the selection is marked afresh
  __syncthreads();
  for (int i = w0; i < w0 + wpt; i += 4) bitmap4[i / 4] = u32x4_t{0u, 0u, 0u, 0u};
  __syncthreads();
  select_emit<kCsaPerT>(key, pos, kCsaPerT, k_eff, S, bitmap4, wpt, out);
}

size_t csa_lds_bytes(int64_t n_cap) {
  const int64_t wpt = (ceil_div64(ceil_div64(n_cap, 32), kSelNT) + 3) / 4 * 4;
  return select_bitmap_lds_bytes(wpt);
}

template <int D>
void km_launch(const KmArgs& k, int rounds, hipStream_t s) {
  hipLaunchKernelGGL(km_init, dim3((unsigned)k.C, (unsigned)k.B), dim3(128), 0, s, k);
  const size_t lds = (size_t)k.C * D * sizeof(float);
  for (int it = 0; it < rounds; ++it) {
    hipLaunchKernelGGL(km_assign<D>, dim3((unsigned)ceil_div64(k.M, 256), (unsigned)k.B), dim3(256),
                       lds, s, k);
    hipLaunchKernelGGL(km_update<D>, dim3((unsigned)k.C, (unsigned)k.B), dim3(256), 0, s, k);
  }
  hipLaunchKernelGGL(km_store, dim3(256), dim3(256), 0, s, k);
}

template <int D>
void csa_launch(const CsaArgs& c, hipStream_t s) {
  hipLaunchKernelGGL(csa_probe<D>, dim3((unsigned)c.B), dim3(256), 0, s, c);
  const int nslot = c.P * c.T + c.nbuf;
  hipLaunchKernelGGL(csa_score<D>, dim3((unsigned)ceil_div64(nslot, 256), (unsigned)c.B), dim3(256),
                     0, s, c);
  hipLaunchKernelGGL(csa_select, dim3((unsigned)c.B), dim3(kSelNT), csa_lds_bytes(c.n_cap), s, c);
}

bool csa_shape_ok(int B, int d, int64_t n_cap, int C, int T) {
  if (B < 1 || B > 65535 || (d != 32 && d != 64 && d != 128)) return false;
  if (n_cap < 1 || n_cap > 524288 || C < 1 || C > kCsaMaxC || T < 1 || T > 2048) return false;
  return (size_t)C * d * sizeof(float) <= 65536;  // the centroids fit the assignment's LDS
}

struct BuildLayout {
  size_t o_mu, o_assign, o_cnt, o_route, total;
};
BuildLayout build_layout(int B, int M, int d, int64_t n_cap, int C, int T) {
  BuildLayout L{};
  size_t o = 0;
  L.o_mu = o; o = align_up(o + (size_t)B * C * d * 4, 256);
  L.o_assign = o; o = align_up(o + (size_t)B * M * 4, 256);
  L.o_cnt = o; o = align_up(o + (size_t)B * C * 4, 256);
  L.o_route = o;
  o = align_up(o + clsa_route_workspace_size(B, C, d, n_cap, T, T, CLSA_BF16), 256);
  L.total = o;
  return L;
}

}  // namespace
}  // namespace clsa

using namespace clsa;

extern "C" size_t clsa_csa_build_workspace_size(int B, int M, int d, int64_t n_cap, int C, int T) {
  if (!csa_shape_ok(B, d, n_cap, C, T) || M < C || (int64_t)B * M > 0x7fffffff) return 0;
  return build_layout(B, M, d, n_cap, C, T).total;
}

extern "C" int clsa_csa_build(const void* q_prefill, const void* K_idx, int B, int M, int d,
                              int64_t n_cap, const int32_t* n_ctx, int C, int rounds, int T,
                              clsa_dtype dt, void* centroids, int32_t* table, void* ws,
                              size_t ws_bytes, void* stream) {
  if (dt != CLSA_BF16) return CLSA_ERR_UNSUPPORTED_DTYPE;
  if (!q_prefill || !K_idx || !centroids || !table) return CLSA_ERR_INVALID;
  if (!csa_shape_ok(B, d, n_cap, C, T) || M < C || rounds < 0 || rounds > 100 ||
      (int64_t)B * M > 0x7fffffff || (int64_t)B * C > 65535)
    return CLSA_ERR_INVALID;
  const BuildLayout L = build_layout(B, M, d, n_cap, C, T);
  if (!ws || ws_bytes < L.total) return CLSA_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  KmArgs k{};
  k.q = static_cast<const uint16_t*>(q_prefill);
  k.B = B;
  k.M = M;
  k.d = d;
  k.C = C;
  k.mu = reinterpret_cast<float*>(w + L.o_mu);
  k.assign = reinterpret_cast<int32_t*>(w + L.o_assign);
  k.cent = static_cast<uint16_t*>(centroids);
  if (d == 32) km_launch<32>(k, rounds, s);
  else if (d == 64) km_launch<64>(k, rounds, s);
  else km_launch<128>(k, rounds, s);
  if (hipGetLastError() != hipSuccess) return CLSA_ERR_HIP;
  // the table: every centroid routed like a query row, k = T
  return clsa_route(centroids, K_idx, B, C, d, n_cap, n_ctx, -1, T, CLSA_BF16, table,
                    reinterpret_cast<int32_t*>(w + L.o_cnt), T, w + L.o_route,
                    ws_bytes - L.o_route, stream);
}

extern "C" size_t clsa_csa_route_workspace_size(int B, int d, int64_t n_cap, int C, int T, int P) {
  if (!csa_shape_ok(B, d, n_cap, C, T) || P < 1 || P > kCsaMaxP || P > C) return 0;
  return align_up((size_t)B * kCsaMaxP * 4, 256) + (size_t)B * kCsaCap * 8;
}

extern "C" int clsa_csa_route(const void* q_idx, const void* K_idx, int B, int d, int64_t n_cap,
                              const int32_t* n_ctx, const void* centroids, const int32_t* table,
                              int C, int T, int64_t n_table, int P, int k, clsa_dtype dt,
                              int32_t* idx, int32_t* counts, int cap, void* ws, size_t ws_bytes,
                              void* stream) {
  if (dt != CLSA_BF16) return CLSA_ERR_UNSUPPORTED_DTYPE;
  if (!q_idx || !K_idx || !centroids || !table || !idx || !counts) return CLSA_ERR_INVALID;
  if (!csa_shape_ok(B, d, n_cap, C, T) || P < 1 || P > kCsaMaxP || P > C || k < 1 || cap < k)
    return CLSA_ERR_INVALID;
  if (n_table < 0 || n_table > n_cap || (int64_t)P * T + (n_cap - n_table) > kCsaCap)
    return CLSA_ERR_INVALID;
  const size_t need = clsa_csa_route_workspace_size(B, d, n_cap, C, T, P);
  if (!ws || ws_bytes < need) return CLSA_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  CsaArgs c{};
  c.q = static_cast<const uint16_t*>(q_idx);
  c.K = static_cast<const uint16_t*>(K_idx);
  c.n_ctx = n_ctx;
  c.cent = static_cast<const uint16_t*>(centroids);
  c.table = table;
  c.n_cap = n_cap;
  c.n_table = n_table;
  c.B = B;
  c.d = d;
  c.C = C;
  c.T = T;
  c.P = P;
  c.k = k;
  c.cap = cap;
  c.nbuf = (int)(n_cap - n_table);
  c.probe = reinterpret_cast<int32_t*>(w);
  c.cand = reinterpret_cast<uint64_t*>(w + align_up((size_t)B * kCsaMaxP * 4, 256));
  c.idx = idx;
  c.counts = counts;
  if (d == 32) csa_launch<32>(c, s);
  else if (d == 64) csa_launch<64>(c, s);
  else csa_launch<128>(c, s);
  return hipGetLastError() == hipSuccess ? CLSA_OK : CLSA_ERR_HIP;
}

// Sparse attention over a shared routing list, all layers in one launch.
//
// Method: CLSA explainer (ai-papers.net), section "CLSAの仕組み" -- every
// cross-decoder layer runs softmax attention over the same routed KV
// positions, produced once per query token.
//
// Grid: (split, row, layer).  A row's index list is cut into ceil(count / TS)
// splits of near-equal length; a split's workgroup writes either the final
// output (one split) or a partial (m, l, acc) that attn_combine merges with
// the log-sum-exp rule.
// No workgroup waits for another; the kernel boundary orders the merge.
//
// attn_bf16  (bf16, D = 64/128/256, Hq/Hkv in {1,2,4,8,16}): one workgroup per
//            KV head and split, four waves over its tokens, in three phases:
//            all scores of the split, an exact softmax over them, then P.V.
//            Every gathered K and V row is read once, as whole cache lines,
//            and used by all G query heads of its KV head.  This is an
//            HBM-bound gather (about 4 flop per byte), so the dot products
//            run on the VALU (v_dot2_f32_bf16) rather than being padded into
//            MFMA tiles.  Loads carry the streaming hint unless the launch's
//            rows share positions (attn_streaming).
// attn_generic (fp32, or shapes attn_bf16 does not take): plain VALU, in
//            sub-blocks of 64 tokens with an online (running max / running
//            sum) softmax.
#include "clsa_common.h"

namespace clsa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kTB = 64;  // tokens per sub-block

struct AttnArgs {
  const void* q[CLSA_MAX_LAYERS];
  const void* K[CLSA_MAX_LAYERS];
  const void* V[CLSA_MAX_LAYERS];
  void* out[CLSA_MAX_LAYERS];
  const int32_t* idx;
  const int32_t* counts;
  float* lse;
  float* pacc;   // [L][R][S][Hq][D]
  float2* pml;   // [L][R][S][Hq]  (running max in log2 units, running sum)
  int64_t n_cap;
  int L, B, M, Hq, Hkv, D, cap, TS, S;
  float scale_log2;  // logit scale times log2(e)
};

CLSA_DEV int row_count(const AttnArgs& a, int r) {
  int c = a.counts[r];
  c = c < 0 ? 0 : c;
  return c > a.cap ? a.cap : c;
}
CLSA_DEV int row_splits(const AttnArgs& a, int cnt) {
  const int s = (cnt + a.TS - 1) / a.TS;
  return s < 1 ? 1 : s;
}
// Entries [begin, end) of split s of a row's cnt entries: the row's nsplit
// splits are as equal as integers allow (each at most TS), so that no
// split of a long row is a short remainder.
CLSA_DEV void split_range(int cnt, int nsplit, int s, int& begin, int& end) {
  begin = (int)(((int64_t)s * cnt) / nsplit);
  end = (int)(((int64_t)(s + 1) * cnt) / nsplit);
}

template <typename T> CLSA_DEV T from_f32(float x);
template <> CLSA_DEV float from_f32<float>(float x) { return x; }
template <> CLSA_DEV uint16_t from_f32<uint16_t>(float x) { return f32_to_bf16(x); }
template <typename T> CLSA_DEV float to_f32(T x);
template <> CLSA_DEV float to_f32<float>(float x) { return x; }
template <> CLSA_DEV float to_f32<uint16_t>(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }

// final (single split) or partial result of one head, from its running state
template <typename T>
CLSA_DEV void emit(const AttnArgs& a, int l, int r, int s, int nsplit, int h, int d, float acc,
                   float m, float lsum, bool write_ml) {
  const size_t orow = ((size_t)r * a.Hq + h) * a.D + d;
  if (nsplit == 1) {
    const float o = lsum > 0.f ? acc / lsum : 0.f;
    static_cast<T*>(a.out[l])[orow] = from_f32<T>(o);
    if (write_ml && a.lse)
      a.lse[((size_t)l * a.B * a.M + r) * a.Hq + h] =
          lsum > 0.f ? (m + __log2f(lsum)) * kLn2 : -INFINITY;
  } else {
    const size_t p = (((size_t)l * a.B * a.M + r) * a.S + s) * a.Hq + h;
    a.pacc[p * a.D + d] = acc;
    if (write_ml) a.pml[p] = make_float2(m, lsum);
  }
}

// ================================================================ combine
// out = sum_s acc_s 2^(m_s - m*) / sum_s l_s 2^(m_s - m*), m* = max_s m_s;
// lse = (m* + log2 sum_s l_s 2^(m_s - m*)) ln 2.  Rows with one split were
// finished by their only workgroup.  One wave per (head, row, layer): a row
// of one sequence has Hq x L of them, enough to spread over the chip.  The
// partials of kCombineGroup splits are loaded together and folded into a
// running maximum and sums, so a row waits on memory once per group.
constexpr int kCombineThreads = 64;
constexpr int kCombineGroup = 8;
constexpr int kCombineDims = 256 / kCombineThreads;  // head dims per lane, D <= 256
template <typename T>
__global__ __launch_bounds__(kCombineThreads) void attn_combine(AttnArgs a) {
  const int h = blockIdx.x, r = blockIdx.y, l = blockIdx.z;
  const int nsplit = row_splits(a, row_count(a, r));
  if (nsplit == 1) return;
  const size_t base = ((size_t)l * a.B * a.M + r) * a.S;
  const int t = threadIdx.x;
  float m = -INFINITY, L = 0.f, o[kCombineDims];
#pragma unroll
  for (int i = 0; i < kCombineDims; ++i) o[i] = 0.f;
  for (int s0 = 0; s0 < nsplit; s0 += kCombineGroup) {
    float2 ml[kCombineGroup];
    float pa[kCombineGroup][kCombineDims];
#pragma unroll
    for (int u = 0; u < kCombineGroup; ++u) {
      const int s = s0 + u;
      const size_t p = (base + s) * a.Hq + h;
      ml[u] = s < nsplit ? a.pml[p] : make_float2(-INFINITY, 0.f);
#pragma unroll
      for (int i = 0; i < kCombineDims; ++i) {
        const int d = t + i * kCombineThreads;
        pa[u][i] = (s < nsplit && d < a.D) ? a.pacc[p * a.D + d] : 0.f;
      }
    }
    float mg = m;
#pragma unroll
    for (int u = 0; u < kCombineGroup; ++u) mg = fmaxf(mg, ml[u].x);
    if (mg == -INFINITY) continue;  // nothing attended so far
    const float keep = m == -INFINITY ? 0.f : exp2f(m - mg);
    L *= keep;
#pragma unroll
    for (int i = 0; i < kCombineDims; ++i) o[i] *= keep;
#pragma unroll
    for (int u = 0; u < kCombineGroup; ++u) {
      const float w = ml[u].x == -INFINITY ? 0.f : exp2f(ml[u].x - mg);
      L = fmaf(ml[u].y, w, L);
#pragma unroll
      for (int i = 0; i < kCombineDims; ++i) o[i] = fmaf(pa[u][i], w, o[i]);
    }
    m = mg;
  }
#pragma unroll
  for (int i = 0; i < kCombineDims; ++i) {
    const int d = t + i * kCombineThreads;
    if (d < a.D)
      static_cast<T*>(a.out[l])[((size_t)r * a.Hq + h) * a.D + d] = from_f32<T>(L > 0.f ? o[i] / L : 0.f);
  }
  if (t == 0 && a.lse)
    a.lse[((size_t)l * a.B * a.M + r) * a.Hq + h] = L > 0.f ? (m + __log2f(L)) * kLn2 : -INFINITY;
}

// ======================================================= gathered (bf16)

// Sum NV per-lane partials over each group of LANES consecutive lanes,
// halving the values kept per lane at each butterfly step while more than
// one is left.  Afterwards v[0 .. max(1, NV/LANES)) hold complete sums of
// value indices base, base+1, ...
template <int NV, int LANES, int M = LANES / 2, int C = NV>
CLSA_DEV void group_reduce(float (&v)[NV], int lane, int& base) {
  if constexpr (M >= 1) {
    if constexpr (C > 1) {
      constexpr int H = C / 2;
      const bool up = (lane & M) != 0;
#pragma unroll
      for (int i = 0; i < H; ++i) {
        const float send = up ? v[i] : v[i + H];
        const float keep = up ? v[i + H] : v[i];
        v[i] = keep + __shfl_xor(send, M);
      }
      base += up ? H : 0;
      group_reduce<NV, LANES, M / 2, H>(v, lane, base);
    } else {
      v[0] += __shfl_xor(v[0], M);
      group_reduce<NV, LANES, M / 2, C>(v, lane, base);
    }
  }
}

constexpr int kWaves = 4;
// scores of one workgroup live in LDS: G heads x TS tokens of fp32
constexpr int kScoreFloats = 8192;
// (at most 2048 tokens, so that groups of one or two query heads still fit
// four workgroups' LDS per CU)
__host__ __device__ constexpr int ts_max(int G) { return kScoreFloats / G < 2048 ? kScoreFloats / G : 2048; }

// Workgroup = (split s, KV head g) x row r x layer l; blockIdx.x = s*Hkv + g.
// Every lane owns 8 consecutive dims (16 bytes) of one token slot, so one
// load instruction reads whole 256-byte K or V rows of 64/(D/8) tokens
// (full cache lines).  NT: streaming hint, for rows read about once per
// launch (decode); without it, rows that many query rows share (a prefill
// chunk) stay in the caches for the next reader.  Three phases, separated by barriers:
//   A  scores: per token, the G query heads' partial dot products over the
//      lane's 8 dims (v_dot2_f32_bf16), reduced across the row's lanes,
//      written to LDS in log2 units (skipped rows -inf);
//   B  softmax: exact per-head max, 2^(s - max) and sum over the split;
//   C  P.V: each gathered V row updates all G heads; the 4 waves' sums
//      meet in LDS.
template <bool NT>
CLSA_DEV u32x4_t load_row16(const uint16_t* p) {
  if constexpr (NT) return load_stream16(p);
  else return *reinterpret_cast<const u32x4_t*>(p);
}

template <int G, int D, bool NT, int AB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(G <= 4 ? 4 : (G <= 8 ? 3 : 2), 8)))
void attn_bf16(AttnArgs a) {
  constexpr int kLPT = D / 8;      // lanes per token row (8 dims each)
  constexpr int kTPW = 64 / kLPT;  // token rows per wave load
  constexpr int kTS = ts_max(G);
  constexpr int kAB = AB;          // K rows in flight per lane
  constexpr int kVB = 4;           // V rows in flight per lane
  constexpr int kNR = G / kLPT > 0 ? G / kLPT : 1;  // sums per lane after the reduce
  constexpr int kShare = kLPT / (G < kLPT ? G : kLPT);  // lanes holding the same sums
  static_assert(G >= 1 && G <= 16 && (G & (G - 1)) == 0, "group size");
  static_assert(D == 64 || D == 128 || D == 256, "head dim");
  static_assert(kWaves * G * D <= kScoreFloats, "wave partials alias the scores");

  __shared__ float sc[G][kTS];     // scores, then probabilities, then wave partials
  __shared__ int sidx[kTS];
  constexpr int kHPW = (G + kWaves - 1) / kWaves;  // heads per wave in phase B

  const int g = blockIdx.x % a.Hkv, s = blockIdx.x / a.Hkv;
  const int r = blockIdx.y, l = blockIdx.z;
  const int lane = lane_id(), w = threadIdx.x / kWave;
  const int cnt = row_count(a, r);
  const int nsplit = row_splits(a, cnt);
  if (s >= nsplit) return;
  int t_begin, t_stop;
  split_range(cnt, nsplit, s, t_begin, t_stop);
  const int nt = t_stop - t_begin;  // tokens of this split, <= TS <= kTS

  const int b = r / a.M;
  const uint16_t* Kl = static_cast<const uint16_t*>(a.K[l]);
  const uint16_t* Vl = static_cast<const uint16_t*>(a.V[l]);
  const uint16_t* ql = static_cast<const uint16_t*>(a.q[l]);
  const int32_t* irow = a.idx + (size_t)r * a.cap + t_begin;
  const size_t head_base = (size_t)b * a.n_cap * a.Hkv + g;  // row j -> (head_base + j*Hkv)*D
  const int tq = lane / kLPT, ds = lane % kLPT;

  for (int i = threadIdx.x; i < nt; i += blockDim.x) {
    const int rw = irow[i];
    sidx[i] = (rw < 0 || (int64_t)rw >= a.n_cap) ? -1 : rw;
  }
  // the lane's 8 dims of every query head of this KV head, as bf16 pairs
  u32x4_t qw[G];
#pragma unroll
  for (int h = 0; h < G; ++h)
    qw[h] = *reinterpret_cast<const u32x4_t*>(ql + (((size_t)r * a.Hq) + g * G + h) * D + ds * 8);
  __syncthreads();

  const int ngroups = (nt + kTPW - 1) / kTPW;
  // V rows of token slots t < nt with a valid position: bit u of vmask
  auto load_v = [&](int grp0, u32x4_t (&vv)[kVB], uint32_t& vmask) {
    vmask = 0u;
#pragma unroll
    for (int u = 0; u < kVB; ++u) {
      const int t = (grp0 + u) * kTPW + tq;
      const int rw = t < nt ? sidx[t] : -1;
      vmask |= rw >= 0 ? 1u << u : 0u;
      vv[u] = load_row16<NT>(Vl + (head_base + (size_t)(rw < 0 ? 0 : rw) * a.Hkv) * D + ds * 8);
    }
  };

  // ---- phase A: scores ----
  for (int grp0 = w * kAB; grp0 < ngroups; grp0 += kWaves * kAB) {
    u32x4_t kk[kAB];
    uint32_t kmask = 0u;  // bit u: slot u holds a valid position
#pragma unroll
    for (int u = 0; u < kAB; ++u) {
      const int t = (grp0 + u) * kTPW + tq;
      const int rw = t < nt ? sidx[t] : -1;
      kmask |= rw >= 0 ? 1u << u : 0u;
      kk[u] = load_row16<NT>(Kl + (head_base + (size_t)(rw < 0 ? 0 : rw) * a.Hkv) * D + ds * 8);
    }
#pragma unroll
    for (int u = 0; u < kAB; ++u) {
      const int t = (grp0 + u) * kTPW + tq;
      float v[G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float acc = dot2(kk[u][0], qw[h][0], 0.f);
        acc = dot2(kk[u][1], qw[h][1], acc);
        acc = dot2(kk[u][2], qw[h][2], acc);
        v[h] = dot2(kk[u][3], qw[h][3], acc);
      }
      int base = 0;
      group_reduce<G, kLPT>(v, lane, base);
      if ((ds & (kShare - 1)) == 0 && t < nt) {
#pragma unroll
        for (int i = 0; i < kNR; ++i)
          sc[base + i][t] = (kmask >> u) & 1u ? v[i] * a.scale_log2 : -INFINITY;
      }
    }
  }
  // The wave's first batch of V rows goes out now and arrives during the
  // softmax rather than after it.  The barriers around the softmax publish
  // LDS only (scores, then probabilities), so they leave these loads in
  // flight.
  u32x4_t vv0[kVB];
  uint32_t vmask0 = 0u;
  const bool first_v = w * kVB < ngroups;  // wave-uniform
  if (first_v) load_v(w * kVB, vv0, vmask0);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

  // ---- phase B: softmax per head over the split; wave w owns heads
  //      w, w+4, ... and keeps their max and sum in registers ----
  float hm[kHPW], hl[kHPW];
#pragma unroll
  for (int i = 0; i < kHPW; ++i) {
    const int h = w + i * kWaves;
    float mx = -INFINITY, sum = 0.f;
    if (h < G) {
      for (int t = lane; t < nt; t += kWave) mx = fmaxf(mx, sc[h][t]);
      mx = wave_max(mx);
      if (mx != -INFINITY) {
        for (int t = lane; t < nt; t += kWave) {
          const float p = exp2f(sc[h][t] - mx);
          sc[h][t] = p;
          sum += p;
        }
      }
      sum = wave_sum(sum);
    }
    hm[i] = mx;
    hl[i] = sum;
  }
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

  // ---- phase C: P.V (skipped rows have p = 0) ----
  float acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  auto fold_v = [&](int grp0, const u32x4_t (&vv)[kVB], uint32_t vmask) {
#pragma unroll
    for (int u = 0; u < kVB; ++u) {
      const int t = (grp0 + u) * kTPW + tq;
      float vf[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vf[2 * e] = bf16_lo(vv[u][e]);
        vf[2 * e + 1] = bf16_hi(vv[u][e]);
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float p = (vmask >> u) & 1u ? sc[h][t] : 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(p, vf[e], acc[h][e]);
      }
    }
  };
  if (first_v) fold_v(w * kVB, vv0, vmask0);
  for (int grp0 = w * kVB + kWaves * kVB; grp0 < ngroups; grp0 += kWaves * kVB) {
    u32x4_t vv[kVB];
    uint32_t vmask;
    load_v(grp0, vv, vmask);
    fold_v(grp0, vv, vmask);
  }
  // sum the token slots sharing a dim slice, then the 4 waves (in LDS)
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v = acc[h][e];
#pragma unroll
      for (int m = kLPT; m < 64; m <<= 1) v += __shfl_xor(v, m);
      acc[h][e] = v;
    }
  __syncthreads();  // every wave is done reading the probabilities
  float* wacc = &sc[0][0];  // [4][G][D]
  if (tq == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) wacc[(w * G + h) * D + ds * 8 + e] = acc[h][e];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kHPW; ++i) {
    const int h = w + i * kWaves;
    if (h < G) {
      for (int d = lane; d < D; d += kWave) {
        float o = 0.f;
#pragma unroll
        for (int v = 0; v < kWaves; ++v) o += wacc[(v * G + h) * D + d];
        emit<uint16_t>(a, l, r, s, nsplit, g * G + h, d, o, hm[i], hl[i], d == 0);
      }
    }
  }
}

// ============================================================ generic VALU
constexpr int kGenMaxPairs = 8192;  // Hq * D
constexpr int kGenMaxHq = 64;

template <typename T>
__global__ __launch_bounds__(256) void attn_generic(AttnArgs a) {
  __shared__ float qs[kGenMaxPairs];
  __shared__ float sc[kGenMaxHq * kTB];
  __shared__ int sidx[kTB];
  __shared__ float m_run[kGenMaxHq], l_run[kGenMaxHq], alpha[kGenMaxHq];

  const int s = blockIdx.x, r = blockIdx.y, l = blockIdx.z;
  const int tid = threadIdx.x;
  const int cnt = row_count(a, r);
  const int nsplit = row_splits(a, cnt);
  if (s >= nsplit) return;
  int t_begin, t_end;
  split_range(cnt, nsplit, s, t_begin, t_end);
  const int b = r / a.M;
  const int Hq = a.Hq, D = a.D, G = a.Hq / a.Hkv;
  const int pairs = Hq * D;
  const T* Kl = static_cast<const T*>(a.K[l]);
  const T* Vl = static_cast<const T*>(a.V[l]);
  const T* ql = static_cast<const T*>(a.q[l]);
  const size_t seq_base = (size_t)b * a.n_cap;

  for (int i = tid; i < pairs; i += 256) qs[i] = to_f32<T>(ql[(size_t)r * pairs + i]);
  for (int h = tid; h < Hq; h += 256) {
    m_run[h] = -INFINITY;
    l_run[h] = 0.f;
  }
  float acc[kGenMaxPairs / 256];
#pragma unroll
  for (int k = 0; k < kGenMaxPairs / 256; ++k) acc[k] = 0.f;
  __syncthreads();

  for (int t0 = t_begin; t0 < t_end; t0 += kTB) {
    const int nt = (t_end - t0) < kTB ? (t_end - t0) : kTB;
    if (tid < kTB) {
      int rw = tid < nt ? a.idx[(size_t)r * a.cap + t0 + tid] : -1;
      if (rw < 0 || (int64_t)rw >= a.n_cap) rw = -1;
      sidx[tid] = rw;
    }
    __syncthreads();
    for (int p = tid; p < Hq * kTB; p += 256) {
      const int h = p / kTB, t = p % kTB;
      float z = -INFINITY;
      if (sidx[t] >= 0) {
        const T* kr = Kl + ((seq_base + sidx[t]) * a.Hkv + h / G) * D;
        float acc_d = 0.f;
        for (int d = 0; d < D; ++d) acc_d = fmaf(qs[h * D + d], to_f32<T>(kr[d]), acc_d);
        z = acc_d * a.scale_log2;
      }
      sc[h * kTB + t] = z;
    }
    __syncthreads();
    for (int h = tid; h < Hq; h += 256) {
      float mx = -INFINITY;
      for (int t = 0; t < kTB; ++t) mx = fmaxf(mx, sc[h * kTB + t]);
      const float m_new = fmaxf(m_run[h], mx);
      float sum = 0.f;
      for (int t = 0; t < kTB; ++t) {
        const float p = (m_new == -INFINITY) ? 0.f : exp2f(sc[h * kTB + t] - m_new);
        sc[h * kTB + t] = p;
        sum += p;
      }
      const float al = (m_new == -INFINITY) ? 1.f : exp2f(m_run[h] - m_new);
      alpha[h] = al;
      l_run[h] = l_run[h] * al + sum;
      m_run[h] = m_new;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kGenMaxPairs / 256; ++k) {
      const int i = tid + k * 256;
      if (i < pairs) {
        const int h = i / D, d = i % D;
        float v = acc[k] * alpha[h];
        for (int t = 0; t < nt; ++t) {
          if (sidx[t] < 0) continue;
          const T* vr = Vl + ((seq_base + sidx[t]) * a.Hkv + h / G) * D;
          v = fmaf(sc[h * kTB + t], to_f32<T>(vr[d]), v);
        }
        acc[k] = v;
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int k = 0; k < kGenMaxPairs / 256; ++k) {
    const int i = tid + k * 256;
    if (i < pairs) {
      const int h = i / D, d = i % D;
      emit<T>(a, l, r, s, nsplit, h, d, acc[k], m_run[h], l_run[h], d == 0);
    }
  }
}

// ================================================================== host
struct Plan {
  bool fast;
  int TS, S;
  size_t o_pml, o_pacc, total;
};

bool attn_shape_ok(int L, int B, int M, int Hq, int Hkv, int D, int cap) {
  if (L < 1 || L > CLSA_MAX_LAYERS || B < 1 || M < 1 || cap < 1) return false;
  if (Hq < 1 || Hkv < 1 || Hkv > 64 || Hq % Hkv != 0 || Hq / Hkv > 16) return false;
  if (D < 8 || D > 256 || D % 8 != 0 || Hq * D > kGenMaxPairs || Hq > kGenMaxHq) return false;
  const int64_t R = (int64_t)B * M;
  if (R > 65535) return false;
  return true;
}

Plan make_plan(int L, int B, int M, int Hq, int Hkv, int D, int cap, clsa_dtype dt) {
  Plan p{};
  const int G = Hq / Hkv;
  p.fast = dt == CLSA_BF16 && (D == 64 || D == 128 || (D == 256 && G <= 8)) &&
           (G == 1 || G == 2 || G == 4 || G == 8 || G == 16);
  const int64_t rows = (int64_t)L * B * M;
  // enough workgroups to fill the chip, without splitting rows needlessly;
  // the bf16 kernel already runs one workgroup per KV head
  const int64_t target = 1024;
  const int64_t per_split = p.fast ? rows * Hkv : rows;
  int64_t S = (target + per_split - 1) / per_split;
  const int64_t min_ts = p.fast ? kTB * kWaves : kTB;
  const int64_t maxS = (cap + min_ts - 1) / min_ts;
  if (S > maxS) S = maxS;
  if (S < 1) S = 1;
  if (p.fast) {  // a split's scores must fit the workgroup's LDS
    const int64_t tsm = ts_max(G);
    const int64_t need = (cap + tsm - 1) / tsm;
    if (S < need) S = need;
  }
  int64_t TS = (cap + S - 1) / S;
  TS = (TS + kTB - 1) / kTB * kTB;
  // Lists longer than a top-k budget (threshold selection) differ in length
  // from row to row: shorter splits spread the long ones over more
  // workgroups (threshold lists of 256 .. 8192 at 128K, 16 layers: 721 us
  // per call unsplit, 471 us with splits of at most 512, 457 us with 768),
  // but no more than 11 per row.  Splits of 1024 measured 487 us: the
  // longest rows' workgroups then form a long tail.
  if (p.fast && cap > 2048) {
    int64_t lim = (cap + 10) / 11;
    lim = (lim + kTB - 1) / kTB * kTB;
    if (lim < 768) lim = 768;
    if (TS > lim) TS = lim;
  }
  p.TS = (int)TS;
  p.S = (int)((cap + TS - 1) / TS);
  size_t o = 0;
  if (p.S > 1) {
    p.o_pml = o;
    o = align_up(o + (size_t)rows * p.S * Hq * sizeof(float2), 256);
    p.o_pacc = o;
    o = align_up(o + (size_t)rows * p.S * Hq * D * sizeof(float), 256);
  }
  p.total = o;
  return p;
}

template <int G, bool NT, int AB>
void launch_fast_gna(int D, dim3 grid, dim3 block, hipStream_t s, const AttnArgs& a) {
  if (D == 128) hipLaunchKernelGGL((attn_bf16<G, 128, NT, AB>), grid, block, 0, s, a);
  else if (D == 64) hipLaunchKernelGGL((attn_bf16<G, 64, NT, AB>), grid, block, 0, s, a);
  else if constexpr (G <= 8) hipLaunchKernelGGL((attn_bf16<G, 256, NT, AB>), grid, block, 0, s, a);
}
// K rows in flight per lane: 4 where a workgroup's split is short (its
// few load rounds are latency-bound: 16 single-layer decode launches 367 ->
// 345 us) or rows share positions (cached loads); 2 for long streaming
// splits, whose loads already keep HBM busy (the 16-layer decode launch is
// 1 % slower with 4).  Issuing a short split's V rows together with its K
// rows (8 K + 4 V per lane) shortened each workgroup by 1 us but not the
// launch (16 single-layer launches 340 us either way; one sequence's
// 16-layer launch 28.3 -> 30.1 us).
template <int G>
void launch_fast_g(int D, bool nt, bool short_split, dim3 grid, dim3 block, hipStream_t s,
                   const AttnArgs& a) {
  if (nt && !short_split) launch_fast_gna<G, true, 2>(D, grid, block, s, a);
  else if (nt) launch_fast_gna<G, true, 4>(D, grid, block, s, a);
  else launch_fast_gna<G, false, 4>(D, grid, block, s, a);
}

// Streaming loads unless a routed K/V row is expected to be read at least
// twice within a layer: a sequence's M query rows pick cap positions each
// out of n_cap.  Measured on a 4096-row prefill chunk at 128K context
// (16 layers, 550 GB gathered): 81 ms with the streaming hint, 65 ms without.
bool attn_streaming(int M, int cap, int64_t n_cap) { return (int64_t)M * cap < 2 * n_cap; }

}  // namespace
}  // namespace clsa

using namespace clsa;

extern "C" size_t clsa_sparse_attn_workspace_size(int L, int B, int M, int Hq, int Hkv, int D,
                                                  int cap, clsa_dtype dt) {
  if (!attn_shape_ok(L, B, M, Hq, Hkv, D, cap)) return 0;
  return make_plan(L, B, M, Hq, Hkv, D, cap, dt).total;
}

extern "C" int clsa_sparse_attn(int L, int B, int M, int Hq, int Hkv, int D,
                                const void* const* q, const void* const* K,
                                const void* const* V, int64_t n_cap, const int32_t* idx,
                                const int32_t* counts, int cap, float scale, clsa_dtype dt,
                                void* const* out, float* lse, void* ws, size_t ws_bytes,
                                void* stream) {
  if (dt != CLSA_F32 && dt != CLSA_BF16) return CLSA_ERR_UNSUPPORTED_DTYPE;
  if (!attn_shape_ok(L, B, M, Hq, Hkv, D, cap) || n_cap < 1) return CLSA_ERR_INVALID;
  if (!q || !K || !V || !out || !idx || !counts) return CLSA_ERR_INVALID;
  for (int l = 0; l < L; ++l)
    if (!q[l] || !K[l] || !V[l] || !out[l]) return CLSA_ERR_INVALID;
  if (!(scale >= 0.f) || scale == INFINITY) return CLSA_ERR_INVALID;
  const Plan p = make_plan(L, B, M, Hq, Hkv, D, cap, dt);
  if (p.total > 0 && (!ws || ws_bytes < p.total)) return CLSA_ERR_WORKSPACE;

  AttnArgs a{};
  for (int l = 0; l < L; ++l) {
    a.q[l] = q[l];
    a.K[l] = K[l];
    a.V[l] = V[l];
    a.out[l] = out[l];
  }
  a.idx = idx;
  a.counts = counts;
  a.lse = lse;
  if (p.S > 1) {
    a.pml = reinterpret_cast<float2*>(static_cast<char*>(ws) + p.o_pml);
    a.pacc = reinterpret_cast<float*>(static_cast<char*>(ws) + p.o_pacc);
  }
  a.n_cap = n_cap;
  a.L = L;
  a.B = B;
  a.M = M;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.D = D;
  a.cap = cap;
  a.TS = p.TS;
  a.S = p.S;
  const float sc = scale > 0.f ? scale : 1.0f / sqrtf((float)D);
  a.scale_log2 = sc * kLog2e;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const int R = B * M;
  const dim3 grid((unsigned)p.S, (unsigned)R, (unsigned)L);
  if (p.fast) {
    const dim3 block(64 * kWaves);
    const dim3 mgrid((unsigned)(p.S * Hkv), (unsigned)R, (unsigned)L);
    const bool nt = attn_streaming(M, cap, n_cap);
    const bool sh = p.S > 1;
    switch (Hq / Hkv) {
      case 1: launch_fast_g<1>(D, nt, sh, mgrid, block, s, a); break;
      case 2: launch_fast_g<2>(D, nt, sh, mgrid, block, s, a); break;
      case 4: launch_fast_g<4>(D, nt, sh, mgrid, block, s, a); break;
      case 8: launch_fast_g<8>(D, nt, sh, mgrid, block, s, a); break;
      default: launch_fast_g<16>(D, nt, sh, mgrid, block, s, a); break;
    }
  } else if (dt == CLSA_BF16) {
    hipLaunchKernelGGL(attn_generic<uint16_t>, grid, dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL(attn_generic<float>, grid, dim3(256), 0, s, a);
  }
  if (p.S > 1) {
    const dim3 cg((unsigned)Hq, (unsigned)R, (unsigned)L);
    if (dt == CLSA_BF16) hipLaunchKernelGGL(attn_combine<uint16_t>, cg, dim3(kCombineThreads), 0, s, a);
    else hipLaunchKernelGGL(attn_combine<float>, cg, dim3(kCombineThreads), 0, s, a);
  }
  return hipGetLastError() == hipSuccess ? CLSA_OK : CLSA_ERR_HIP;
}

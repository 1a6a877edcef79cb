// Sparse attention over a shared routing list, all layers in one launch.
//
// Method: CLSA explainer (ai-papers.net), section "CLSAの仕組み" -- every
// cross-decoder layer runs softmax attention over the same routed KV
// positions, produced once per query token.
//
// Grid: (split, row, layer).  A split is TS consecutive entries of the row's
// index list; each workgroup streams its entries in sub-blocks of 64
// tokens with an online (running max / running sum) softmax and writes
// either the final output (one split) or a partial (m, l, acc).  The last
// split workgroup of a (layer, row) to arrive merges the partials with the
// log-sum-exp rule (combine_row); no workgroup waits for another.
//
// attn_mfma  (bf16, D = 64/128, Hq/Hkv <= 16): one wave per KV head.  The
//            scores of the G query heads of that KV head against 16 gathered
//            key rows are one v_mfma_f32_16x16x32_bf16 chain: the A operand is
//            the G query rows (zero-padded to 16), the B operand is 16 bytes
//            of each key row per lane, loaded straight from HBM.  P.V runs on
//            the VALU: each lane owns 8 consecutive output dims of one token
//            slot and accumulates all G heads, so every gathered V byte is
//            read once and used G times.
// attn_generic (fp32, or shapes the MFMA kernel does not take): plain VALU.
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
  uint32_t* ticket;  // [L][R] arrivals of split workgroups (zeroed per call)
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
// lse = (m* + log2 sum_s l_s 2^(m_s - m*)) ln 2.  Run by the last split
// workgroup of (l, r) after an acquire fence.
template <typename T>
CLSA_DEV void combine_row(const AttnArgs& a, int l, int r, int nsplit) {
  const size_t base = ((size_t)l * a.B * a.M + r) * a.S;
  for (int i = threadIdx.x; i < a.Hq * a.D; i += blockDim.x) {
    const int h = i / a.D, d = i % a.D;
    float ms = -INFINITY;
    for (int s = 0; s < nsplit; ++s) ms = fmaxf(ms, a.pml[(base + s) * a.Hq + h].x);
    float L = 0.f, o = 0.f;
    if (ms != -INFINITY) {
      for (int s = 0; s < nsplit; ++s) {
        const float2 ml = a.pml[(base + s) * a.Hq + h];
        const float wgt = (ml.x == -INFINITY) ? 0.f : exp2f(ml.x - ms);
        L = fmaf(ml.y, wgt, L);
        o = fmaf(a.pacc[((base + s) * a.Hq + h) * a.D + d], wgt, o);
      }
    }
    const float res = L > 0.f ? o / L : 0.f;
    static_cast<T*>(a.out[l])[((size_t)r * a.Hq + h) * a.D + d] = from_f32<T>(res);
    if (d == 0 && a.lse)
      a.lse[((size_t)l * a.B * a.M + r) * a.Hq + h] = L > 0.f ? (ms + __log2f(L)) * kLn2 : -INFINITY;
  }
}

// Called by every thread of a split workgroup after its partial is written.
template <typename T>
CLSA_DEV void finish_split(const AttnArgs& a, int l, int r, int nsplit, uint32_t* s_last) {
  if (nsplit == 1) return;
  __syncthreads();
  if (threadIdx.x == 0)
    *s_last = (arrive_release(&a.ticket[(size_t)l * a.B * a.M + r]) == (uint32_t)(nsplit - 1));
  __syncthreads();
  if (!*s_last) return;
  acquire_device();
  combine_row<T>(a, l, r, nsplit);
}

// ============================================================ MFMA (bf16)
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

template <int G, int D>
__global__ __launch_bounds__(512) void attn_mfma(AttnArgs a) {
  constexpr int kSteps = D / 32;   // MFMA k-steps (32 dims each)
  constexpr int kQuarter = D / 4;  // dims owned by one k-block of lanes
  constexpr int kLPT = D / 8;      // PV lanes per token (8 dims each)
  constexpr int kTPW = 64 / kLPT;  // PV tokens per wave pass
  static_assert(G >= 1 && G <= 16, "group size");
  static_assert(D == 64 || D == 128, "head dim");

  __shared__ float sc_all[8][G][kTB];
  __shared__ uint32_t s_last;

  const int s = blockIdx.x, r = blockIdx.y, l = blockIdx.z;
  const int lane = lane_id(), w = threadIdx.x / kWave;
  const int W = blockDim.x / kWave;
  const int cnt = row_count(a, r);
  const int nsplit = row_splits(a, cnt);
  if (s >= nsplit) return;
  const int t_begin = s * a.TS;
  int t_end = t_begin + a.TS;
  t_end = t_end < cnt ? t_end : cnt;

  const int b = r / a.M;
  float (*sc)[kTB] = sc_all[w];
  const uint16_t* Kl = static_cast<const uint16_t*>(a.K[l]);
  const uint16_t* Vl = static_cast<const uint16_t*>(a.V[l]);
  const uint16_t* ql = static_cast<const uint16_t*>(a.q[l]);
  const int32_t* irow = a.idx + (size_t)r * a.cap;
  const size_t seq_base = (size_t)b * a.n_cap;

  const int kb = lane / 16, col = lane % 16;  // MFMA lane coordinates
  const int tq = lane / kLPT, ds = lane % kLPT;  // PV lane coordinates

  for (int g = w; g < a.Hkv; g += W) {
    // A operand: query rows of this KV head's group, zero beyond G
    bf16x8_t qa[kSteps];
#pragma unroll
    for (int st = 0; st < kSteps; ++st) {
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (col < G) {
        const size_t qo = (((size_t)r * a.Hq) + g * G + col) * D + kb * kQuarter + st * 8;
        v = *reinterpret_cast<const u32x4_t*>(ql + qo);
      }
      qa[st] = __builtin_bit_cast(bf16x8_t, v);
    }
    float m_run[G], l_run[G], acc[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      m_run[h] = -INFINITY;
      l_run[h] = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
    }

    for (int t0 = t_begin; t0 < t_end; t0 += kTB) {
      const int nt = (t_end - t0) < kTB ? (t_end - t0) : kTB;
      int myrow = -1;
      if (lane < nt) myrow = irow[t0 + lane];
      if (myrow < 0 || (int64_t)myrow >= a.n_cap) myrow = -1;

      // ---- scores: 4 tiles of 16 tokens, one MFMA chain per tile ----
      u32x4_t kv[4][kSteps];
#pragma unroll
      for (int tile = 0; tile < 4; ++tile) {
        const int rw = __shfl(myrow, tile * 16 + col);
        const size_t ro = ((seq_base + (size_t)(rw < 0 ? 0 : rw)) * a.Hkv + g) * D + kb * kQuarter;
#pragma unroll
        for (int st = 0; st < kSteps; ++st)
          kv[tile][st] = *reinterpret_cast<const u32x4_t*>(Kl + ro + st * 8);
      }
#pragma unroll
      for (int tile = 0; tile < 4; ++tile) {
        f32x4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < kSteps; ++st)
          c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[st],
                                                      __builtin_bit_cast(bf16x8_t, kv[tile][st]),
                                                      c, 0, 0, 0);
        const int rw = __shfl(myrow, tile * 16 + col);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int h = kb * 4 + j;
          if (h < G) sc[h][tile * 16 + col] = rw >= 0 ? c[j] * a.scale_log2 : -INFINITY;
        }
      }
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");

      // ---- online softmax, lane = token ----
      float alpha[G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float v = sc[h][lane];
        const float mx = wave_max(v);
        const float m_new = fmaxf(m_run[h], mx);
        const float p = (m_new == -INFINITY) ? 0.f : exp2f(v - m_new);
        const float sum = wave_sum(p);
        alpha[h] = (m_new == -INFINITY) ? 1.f : exp2f(m_run[h] - m_new);
        l_run[h] = l_run[h] * alpha[h] + sum;
        m_run[h] = m_new;
        sc[h][lane] = p;
      }
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");

      // ---- P.V: lane owns dims ds*8..ds*8+7 of tokens tq, tq+kTPW, ... ----
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] *= alpha[h];
#pragma unroll 4
      for (int i = 0; i < kTB / kTPW; ++i) {
        const int t = tq + i * kTPW;
        const int rw = __shfl(myrow, t);
        const size_t ro = ((seq_base + (size_t)(rw < 0 ? 0 : rw)) * a.Hkv + g) * D + ds * 8;
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(Vl + ro);
        float vf[8];
        vf[0] = bf16_lo(v[0]); vf[1] = bf16_hi(v[0]);
        vf[2] = bf16_lo(v[1]); vf[3] = bf16_hi(v[1]);
        vf[4] = bf16_lo(v[2]); vf[5] = bf16_hi(v[2]);
        vf[6] = bf16_lo(v[3]); vf[7] = bf16_hi(v[3]);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float p = sc[h][t];
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(p, vf[e], acc[h][e]);
        }
      }
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    }

    // reduce the kTPW token slots that share a dim slice
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float v = acc[h][e];
#pragma unroll
        for (int m = kLPT; m < 64; m <<= 1) v += __shfl_xor(v, m);
        acc[h][e] = v;
      }
    if (tq == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          emit<uint16_t>(a, l, r, s, nsplit, g * G + h, ds * 8 + e, acc[h][e], m_run[h],
                         l_run[h], ds == 0 && e == 0);
    }
  }
  finish_split<uint16_t>(a, l, r, nsplit, &s_last);
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
  __shared__ uint32_t s_last;

  const int s = blockIdx.x, r = blockIdx.y, l = blockIdx.z;
  const int tid = threadIdx.x;
  const int cnt = row_count(a, r);
  const int nsplit = row_splits(a, cnt);
  if (s >= nsplit) return;
  const int t_begin = s * a.TS;
  int t_end = t_begin + a.TS;
  t_end = t_end < cnt ? t_end : cnt;
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
  finish_split<T>(a, l, r, nsplit, &s_last);
}

// ================================================================== host
struct Plan {
  bool mfma;
  int TS, S, W;
  size_t o_ticket, ticket_bytes, o_pml, o_pacc, total;
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
  p.mfma = dt == CLSA_BF16 && (D == 64 || D == 128) &&
           (G == 1 || G == 2 || G == 4 || G == 8 || G == 16);
  p.W = Hkv < 8 ? Hkv : 8;
  const int64_t rows = (int64_t)L * B * M;
  // enough workgroups to fill the chip, without splitting rows needlessly
  const int64_t target = 1024;
  int64_t S = (target + rows - 1) / rows;
  const int64_t maxS = (cap + kTB - 1) / kTB;
  if (S > maxS) S = maxS;
  if (S < 1) S = 1;
  int64_t TS = (cap + S - 1) / S;
  TS = (TS + kTB - 1) / kTB * kTB;
  p.TS = (int)TS;
  p.S = (int)((cap + TS - 1) / TS);
  size_t o = 0;
  if (p.S > 1) {
    p.o_ticket = o;
    p.ticket_bytes = align_up((size_t)rows * 4, 256);
    o += p.ticket_bytes;
    p.o_pml = o;
    o = align_up(o + (size_t)rows * p.S * Hq * sizeof(float2), 256);
    p.o_pacc = o;
    o = align_up(o + (size_t)rows * p.S * Hq * D * sizeof(float), 256);
  }
  p.total = o;
  return p;
}

template <int G>
void launch_mfma_g(int D, dim3 grid, dim3 block, hipStream_t s, const AttnArgs& a) {
  if (D == 128) hipLaunchKernelGGL((attn_mfma<G, 128>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((attn_mfma<G, 64>), grid, block, 0, s, a);
}

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
    a.ticket = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + p.o_ticket);
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
  if (p.S > 1 && zero_fill(a.ticket, p.ticket_bytes, s) != hipSuccess) return CLSA_ERR_HIP;
  const dim3 grid((unsigned)p.S, (unsigned)R, (unsigned)L);
  if (p.mfma) {
    const dim3 block((unsigned)(64 * p.W));
    switch (Hq / Hkv) {
      case 1: launch_mfma_g<1>(D, grid, block, s, a); break;
      case 2: launch_mfma_g<2>(D, grid, block, s, a); break;
      case 4: launch_mfma_g<4>(D, grid, block, s, a); break;
      case 8: launch_mfma_g<8>(D, grid, block, s, a); break;
      default: launch_mfma_g<16>(D, grid, block, s, a); break;
    }
  } else if (dt == CLSA_BF16) {
    hipLaunchKernelGGL(attn_generic<uint16_t>, grid, dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL(attn_generic<float>, grid, dim3(256), 0, s, a);
  }
  return hipGetLastError() == hipSuccess ? CLSA_OK : CLSA_ERR_HIP;
}

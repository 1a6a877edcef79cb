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

}  // namespace clsa

// Host helpers implemented in clsa_api.hip.
namespace clsa {
// Zero `bytes` (multiple of 4) at `p` with a fill kernel on `stream`.
hipError_t zero_fill(void* p, size_t bytes, hipStream_t stream);
inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
}  // namespace clsa

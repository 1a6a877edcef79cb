// libclsa: version, status strings and the workspace fill kernel.
#include "clsa_common.h"

namespace clsa {

__global__ __launch_bounds__(256) void fill_zero_kernel(uint4* p, size_t n16, uint32_t* tail,
                                                        size_t ntail) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
  if (blockIdx.x == 0 && threadIdx.x < ntail) tail[threadIdx.x] = 0u;
}

hipError_t zero_fill(void* p, size_t bytes, hipStream_t stream) {
  if (bytes == 0) return hipSuccess;
  const size_t n16 = bytes / 16;
  const size_t ntail = (bytes % 16) / 4;
  uint32_t* tail = reinterpret_cast<uint32_t*>(static_cast<char*>(p) + n16 * 16);
  size_t blocks = (n16 + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  if (blocks == 0) blocks = 1;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     static_cast<uint4*>(p), n16, tail, ntail);
  return hipGetLastError();
}

struct AppendArgs {
  const void* src[2 * CLSA_MAX_LAYERS + 1];
  void* dst[2 * CLSA_MAX_LAYERS + 1];
  const int32_t* pos;
  int64_t n_cap;
  int B;
  int row_bytes_kv;   // Hkv * D * esize
  int row_bytes_idx;  // d * esize
  int n_kv;           // 2 * L
};

// blockIdx.x = tensor (K0, V0, K1, V1, ..., then the routing keys), y = sequence
__global__ __launch_bounds__(128) void kv_append_kernel(AppendArgs a) {
  const int t = blockIdx.x, b = blockIdx.y;
  const int rb = t < a.n_kv ? a.row_bytes_kv : a.row_bytes_idx;
  const int nv = rb / 16;
  const uint4* src = reinterpret_cast<const uint4*>(static_cast<const char*>(a.src[t]) +
                                                    (size_t)b * rb);
  // the row's first 16-byte pieces are requested together with the slot, so
  // the copy waits on memory once
  const bool first = (int)threadIdx.x < nv;
  const uint4 v0 = first ? src[threadIdx.x] : uint4{};
  const int p = a.pos[b];
  if (p < 0 || (int64_t)p >= a.n_cap) return;
  uint4* dst = reinterpret_cast<uint4*>(static_cast<char*>(a.dst[t]) +
                                        ((size_t)b * a.n_cap + p) * rb);
  if (first) dst[threadIdx.x] = v0;
  for (int i = threadIdx.x + blockDim.x; i < nv; i += blockDim.x) dst[i] = src[i];
}

}  // namespace clsa

extern "C" int clsa_kv_append(int L, int B, int Hkv, int D, int d, int64_t n_cap,
                              const int32_t* pos, const void* src_idx, void* dst_idx,
                              const void* const* src_k, void* const* K,
                              const void* const* src_v, void* const* V, clsa_dtype dt,
                              void* stream) {
  using namespace clsa;
  if (dt != CLSA_F32 && dt != CLSA_BF16) return CLSA_ERR_UNSUPPORTED_DTYPE;
  if (L < 0 || L > CLSA_MAX_LAYERS || B < 1 || B > 65535 || n_cap < 1 || !pos)
    return CLSA_ERR_INVALID;
  const int es = dt == CLSA_BF16 ? 2 : 4;
  if ((src_idx == nullptr) != (dst_idx == nullptr)) return CLSA_ERR_INVALID;
  if (src_idx && (d < 1 || (d * es) % 16 != 0)) return CLSA_ERR_INVALID;
  if (L > 0 && (Hkv < 1 || D < 1 || ((int64_t)Hkv * D * es) % 16 != 0 || !src_k || !K ||
                !src_v || !V))
    return CLSA_ERR_INVALID;
  AppendArgs a{};
  int n = 0;
  for (int l = 0; l < L; ++l) {
    if (!src_k[l] || !K[l] || !src_v[l] || !V[l]) return CLSA_ERR_INVALID;
    a.src[n] = src_k[l];
    a.dst[n++] = K[l];
    a.src[n] = src_v[l];
    a.dst[n++] = V[l];
  }
  a.n_kv = n;
  if (src_idx) {
    a.src[n] = src_idx;
    a.dst[n++] = dst_idx;
  }
  if (n == 0) return CLSA_OK;
  a.pos = pos;
  a.n_cap = n_cap;
  a.B = B;
  a.row_bytes_kv = Hkv * D * es;
  a.row_bytes_idx = d * es;
  hipLaunchKernelGGL(kv_append_kernel, dim3((unsigned)n, (unsigned)B), dim3(128), 0,
                     static_cast<hipStream_t>(stream), a);
  return hipGetLastError() == hipSuccess ? CLSA_OK : CLSA_ERR_HIP;
}

extern "C" int clsa_version(void) { return CLSA_VERSION; }

extern "C" const char* clsa_status_string(int status) {
  switch (status) {
    case CLSA_OK: return "ok";
    case CLSA_ERR_INVALID: return "invalid argument";
    case CLSA_ERR_WORKSPACE: return "workspace too small";
    case CLSA_ERR_UNSUPPORTED_DTYPE: return "unsupported dtype";
    case CLSA_ERR_HIP: return "HIP launch failure";
    case CLSA_ERR_SCRATCH_LIMIT: return "shapes exceed the static scratch array";
    default: return "unknown status";
  }
}

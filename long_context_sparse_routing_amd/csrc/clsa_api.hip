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

}  // namespace clsa

extern "C" int clsa_version(void) { return CLSA_VERSION; }

extern "C" const char* clsa_status_string(int status) {
  switch (status) {
    case CLSA_OK: return "ok";
    case CLSA_ERR_INVALID: return "invalid argument";
    case CLSA_ERR_WORKSPACE: return "workspace too small";
    case CLSA_ERR_UNSUPPORTED_DTYPE: return "unsupported dtype";
    case CLSA_ERR_HIP: return "HIP launch failure";
    default: return "unknown status";
  }
}

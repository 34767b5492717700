// Small utility kernels: workspace clearing (a fill kernel rather than a
// memset node, so the calls stay safe under stream capture).
#include "internal.h"

namespace pr {

__global__ void k_zero(uint4 *p, size_t n16, unsigned char *tail, size_t ntail) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) p[i] = make_uint4(0, 0, 0, 0);
  if (blockIdx.x == 0 && threadIdx.x < ntail) tail[threadIdx.x] = 0;
}

hipError_t launch_zero(void *p, size_t bytes, hipStream_t s) {
  if (bytes == 0) return hipSuccess;
  const size_t n16 = bytes / 16, ntail = bytes % 16;
  size_t blocks = (n16 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks == 0) blocks = 1;
  hipLaunchKernelGGL(k_zero, dim3((unsigned)blocks), dim3(256), 0, s, (uint4 *)p, n16,
                     (unsigned char *)p + n16 * 16, ntail);
  return hipGetLastError();
}

}  // namespace pr

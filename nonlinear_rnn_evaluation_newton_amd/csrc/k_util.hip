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

// dst[c][r] = src[r][c] for a row-major [R, C] matrix of 2- or 4-byte
// elements, through 64 x 64 LDS tiles (coalesced reads along C and writes
// along R).  Turns the K-outer operands of the adjoint's products into the
// K-contiguous layout the GEMM's fast path reads.
template <typename E>
__global__ __launch_bounds__(256) void k_transpose(const E *__restrict__ src, E *__restrict__ dst, int R, int C) {
  __shared__ E tile[64][65];
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64;
#pragma unroll
  for (int i = ty; i < 64; i += 4)
    if (r0 + i < R && c0 + tx < C) tile[i][tx] = src[(size_t)(r0 + i) * C + c0 + tx];
  __syncthreads();
#pragma unroll
  for (int i = ty; i < 64; i += 4)
    if (c0 + i < C && r0 + tx < R) dst[(size_t)(c0 + i) * R + r0 + tx] = tile[tx][i];
}

hipError_t launch_transpose(const void *src, void *dst, int R, int C, int elem_bytes, hipStream_t s) {
  if (R <= 0 || C <= 0) return hipSuccess;
  const dim3 grid((unsigned)((C + 63) / 64), (unsigned)((R + 63) / 64));
  if (grid.y > 65535u) return hipErrorInvalidValue;
  if (elem_bytes == 2)
    hipLaunchKernelGGL(k_transpose<uint16_t>, grid, dim3(256), 0, s, (const uint16_t *)src, (uint16_t *)dst, R, C);
  else if (elem_bytes == 4)
    hipLaunchKernelGGL(k_transpose<float>, grid, dim3(256), 0, s, (const float *)src, (float *)dst, R, C);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pr

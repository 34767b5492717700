// Small utility kernels: workspace clearing (a fill kernel rather than a
// memset node, so the calls stay safe under stream capture).
#include "internal.h"
#include "cells_chan.h"

namespace pr {

__global__ void k_zero(uint4 *p, size_t n16, unsigned char *tail, size_t ntail) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) p[i] = make_uint4(0, 0, 0, 0);
  if (blockIdx.x == 0 && threadIdx.x < ntail) tail[threadIdx.x] = 0;
}

__global__ __launch_bounds__(256) void k_snapshot(const unsigned *src, unsigned *dst, int nwords, unsigned *seq,
                                                  unsigned val) {
  for (int i = threadIdx.x; i < nwords; i += blockDim.x) dst[i] = src[i];
  __threadfence_system();
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_store(seq, val, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
}

hipError_t launch_snapshot(const void *src, void *dst, size_t bytes, unsigned *seq, unsigned val, hipStream_t s) {
  hipLaunchKernelGGL(k_snapshot, dim3(1), dim3(256), 0, s, (const unsigned *)src, (unsigned *)dst, (int)(bytes / 4),
                     seq, val);
  return hipGetLastError();
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

// out[0, 3n) = scale_g (b_x + b_h folded), out[3n, 6n) = scale_g, g = i / n
template <typename ST>
__global__ void k_fold_bias(const ST *bx, const ST *bh, int n, int folded, float g0, float g1, float g2,
                            float *out) {
  const int total = 3 * n;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < total; i += gridDim.x * blockDim.x) {
    const int gate = i / n;
    const float v = bx ? ldf(bx, i) : 0.f;
    const float sc = gate == 0 ? g0 : gate == 1 ? g1 : g2;
    out[i] = sc * ((bh && gate < folded) ? v + ldf(bh, i) : v);
    out[total + i] = sc;
  }
}

hipError_t launch_fold_bias(bool bf16, const void *bx, const void *bh, int n, int cell, float *out, hipStream_t s) {
  const int blocks = (3 * n + 255) / 256 < 1024 ? (3 * n + 255) / 256 : 1024;
  const int folded = cell == C_LSTM ? 3 : 2;
  const float g0 = chan_gate_scale(cell, 0), g1 = chan_gate_scale(cell, 1), g2 = chan_gate_scale(cell, 2);
  if (bf16)
    hipLaunchKernelGGL(k_fold_bias<uint16_t>, dim3(blocks), dim3(256), 0, s, (const uint16_t *)bx,
                       (const uint16_t *)bh, n, folded, g0, g1, g2, out);
  else
    hipLaunchKernelGGL(k_fold_bias<float>, dim3(blocks), dim3(256), 0, s, (const float *)bx, (const float *)bh, n,
                       folded, g0, g1, g2, out);
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

// The same for 2-byte elements with 16-byte accesses on both sides (R and C
// multiples of 8, 16-byte aligned matrices): a thread loads 8 adjacent
// elements of a row, the tile sits in LDS with chunk c8 of row r at chunk
// c8 ^ ((r / 8) % 8) (the 8 rows r8, r8 + 8, ... read together for one
// output chunk fall in distinct banks), and a thread gathers 8 adjacent
// rows of one column into one 16-byte store.
__global__ __launch_bounds__(256) void k_transpose16(const uint16_t *__restrict__ src, uint16_t *__restrict__ dst,
                                                     int R, int C) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[64 * 64];
  const int tid = threadIdx.x;
  const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64;
#pragma unroll
  for (int q = 0; q < 2; q++) {
    const int e = tid + 256 * q, r = e >> 3, ch = e & 7;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (r0 + r < R && c0 + ch * 8 < C) v = *reinterpret_cast<const uint4 *>(src + (size_t)(r0 + r) * C + c0 + ch * 8);
    *reinterpret_cast<uint4 *>(&tile[r * 64 + ((ch ^ ((r >> 3) & 7)) * 8)]) = v;
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 2; q++) {
    const int e = tid + 256 * q, cc = e >> 3, r8 = (e & 7) * 8;
    unsigned w[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int ra = r8 + 2 * i, rb = ra + 1;
      const unsigned lo = tile[ra * 64 + (((cc >> 3) ^ ((ra >> 3) & 7)) * 8) + (cc & 7)];
      const unsigned hi = tile[rb * 64 + (((cc >> 3) ^ ((rb >> 3) & 7)) * 8) + (cc & 7)];
      w[i] = lo | (hi << 16);
    }
    if (c0 + cc < C && r0 + r8 < R)
      *reinterpret_cast<uint4 *>(dst + (size_t)(c0 + cc) * R + r0 + r8) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

hipError_t launch_transpose(const void *src, void *dst, int R, int C, int elem_bytes, hipStream_t s) {
  if (R <= 0 || C <= 0) return hipSuccess;
  if (elem_bytes == 2 && R % 8 == 0 && C % 8 == 0 && ((uintptr_t)src % 16) == 0 && ((uintptr_t)dst % 16) == 0) {
    const dim3 grid((unsigned)((C + 63) / 64), (unsigned)((R + 63) / 64));
    if (grid.y > 65535u) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_transpose16, grid, dim3(256), 0, s, (const uint16_t *)src, (uint16_t *)dst, R, C);
    return hipGetLastError();
  }
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

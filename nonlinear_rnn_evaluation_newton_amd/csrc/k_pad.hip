// Zero-padding of a dense GRU's weights and states to the n = 64 kernels'
// width, and the copies back.  Gate-blocked matrices [G * n, cols] become
// [G * np, cols_p]: row g * np + j holds row g * n + j of the source for
// j < n (its first cols columns), zeros elsewhere.  With only_gate >= 0 the
// source is a single gate [n, cols] that fills gate block only_gate of the
// G blocks, the others zero (a tanh RNN's weights as a GRU's candidate
// gate).  State-like arrays [rows, n] become [rows, np] the same way.  fp32
// throughout.
#include "internal.h"

namespace pr {

__global__ void k_pad_gates(const float *__restrict__ src, int G, int n, int cols, float *__restrict__ dst, int np,
                            int cols_p, int only_gate) {
  const long long total = (long long)G * np * cols_p;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (long long)gridDim.x * blockDim.x) {
    const int c = (int)(i % cols_p);
    const long long r = i / cols_p;
    const int g = (int)(r / np), j = (int)(r % np);
    const bool take = j < n && c < cols && (only_gate < 0 || g == only_gate);
    dst[i] = take ? src[((long long)(only_gate < 0 ? g : 0) * n + j) * cols + c] : 0.f;
  }
}

// dst[g * np + j] = v[g] for j < n and the first two gate blocks (g = 0, 1)
__global__ void k_gate_consts(float *__restrict__ dst, int n, int np, float v0, float v1) {
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j < n) {
    dst[j] = v0;
    dst[np + j] = v1;
  }
}

__global__ void k_unpad_gates(const float *__restrict__ src, int G, int n, int cols, float *__restrict__ dst, int np,
                              int cols_p) {
  const long long total = (long long)G * n * cols;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (long long)gridDim.x * blockDim.x) {
    const int c = (int)(i % cols);
    const long long r = i / cols;
    const int g = (int)(r / n), j = (int)(r % n);
    dst[i] = src[((long long)g * np + j) * cols_p + c];
  }
}

static unsigned pad_blocks(long long total) {
  long long b = (total + 255) / 256;
  if (b > 8192) b = 8192;
  return (unsigned)(b < 1 ? 1 : b);
}

hipError_t launch_pad_gates(const float *src, int G, int n, int cols, float *dst, int np, int cols_p, hipStream_t s,
                            int only_gate) {
  hipLaunchKernelGGL(k_pad_gates, dim3(pad_blocks((long long)G * np * cols_p)), dim3(256), 0, s, src, G, n, cols, dst,
                     np, cols_p, only_gate);
  return hipGetLastError();
}

hipError_t launch_gate_consts(float *dst, int n, int np, float v0, float v1, hipStream_t s) {
  hipLaunchKernelGGL(k_gate_consts, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, dst, n, np, v0, v1);
  return hipGetLastError();
}

hipError_t launch_unpad_gates(const float *src, int G, int n, int cols, float *dst, int np, int cols_p,
                              hipStream_t s) {
  hipLaunchKernelGGL(k_unpad_gates, dim3(pad_blocks((long long)G * n * cols)), dim3(256), 0, s, src, G, n, cols, dst,
                     np, cols_p);
  return hipGetLastError();
}

}  // namespace pr

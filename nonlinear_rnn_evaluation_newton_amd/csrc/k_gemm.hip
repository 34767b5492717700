// MFMA GEMM for the dense contractions of the path: the input projection
// U = x W_x^T + b_x, done once per solve, and the adjoint's dx = dU W_x and
// dW_x = dU^T x.  C[M,N] = sum_k A[m,k] B[n,k] with either operand stored
// K-contiguous or M/N-contiguous, bf16 inputs on v_mfma_f32_32x32x16_bf16 or
// fp32 inputs on v_mfma_f32_32x32x2_f32, fp32 accumulation.
//
// Tiling: 128 x 128 block tile, K step 32, 4 wavefronts of 64 x 64 (2 x 2
// MFMA tiles of 32 x 32), LDS double buffer holding both operands
// K-contiguous so every lane reads its MFMA operand with one vector load.
// Long-K products (dW_x) split K over blocks into an fp32 workspace that a
// second kernel sums in a fixed order.
#include "internal.h"

namespace pr {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

template <typename T>
struct Mfma;
template <>
struct Mfma<uint16_t> {
  static constexpr int KSTEP = 16, VEC = 8;
  __device__ static inline f32x16_t mma(const uint16_t *a, const uint16_t *b, f32x16_t c) {
    bf16x8_t va = *reinterpret_cast<const bf16x8_t *>(a);
    bf16x8_t vb = *reinterpret_cast<const bf16x8_t *>(b);
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, vb, c, 0, 0, 0);
  }
};
template <>
struct Mfma<float> {
  static constexpr int KSTEP = 2, VEC = 1;
  __device__ static inline f32x16_t mma(const float *a, const float *b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(*a, *b, c, 0, 0, 0);
  }
};

constexpr int GBM = 128, GBN = 128, GBK = 32;

template <typename T>
struct GemmLds {
  static constexpr int PAD = 16 / sizeof(T);  // keeps row starts off one bank
  static constexpr int LD = GBK + PAD;
};

// Load one 128 x 32 operand tile (rows r0.., k0..) from global into registers:
// KC: element (r, k) at P[r * ld + k]; else at P[k * ld + r].
template <typename T, bool KC>
struct TileLoader {
  static constexpr int VE = 16 / sizeof(T);                 // elements per 16-byte vector
  static constexpr int NV = GBM * GBK / VE / 256;           // vectors per thread
  uint4 v[NV];
  __device__ inline void load(const T *P, int ld, int rows, int K, int r0, int k0, bool vec) {
#pragma unroll
    for (int q = 0; q < NV; q++) {
      const int e = threadIdx.x + q * 256;
      int r, k;
      if (KC) { r = e / (GBK / VE); k = (e % (GBK / VE)) * VE; }
      else { k = e / (GBM / VE); r = (e % (GBM / VE)) * VE; }
      const int gr = r0 + r, gk = k0 + k;
      T tmp[VE];
      const bool full = KC ? (gr < rows && gk + VE <= K) : (gk < K && gr + VE <= rows);
      if (vec && full) {
        v[q] = *reinterpret_cast<const uint4 *>(KC ? P + (size_t)gr * ld + gk : P + (size_t)gk * ld + gr);
        continue;
      }
#pragma unroll
      for (int i = 0; i < VE; i++) {
        const int rr = KC ? gr : gr + i, kk = KC ? gk + i : gk;
        tmp[i] = (rr < rows && kk < K) ? (KC ? P[(size_t)rr * ld + kk] : P[(size_t)kk * ld + rr]) : (T)0;
      }
      v[q] = *reinterpret_cast<const uint4 *>(tmp);
    }
  }
  __device__ inline void store(T *S) const {
#pragma unroll
    for (int q = 0; q < NV; q++) {
      const int e = threadIdx.x + q * 256;
      if (KC) {
        const int r = e / (GBK / VE), k = (e % (GBK / VE)) * VE;
        *reinterpret_cast<uint4 *>(S + r * GemmLds<T>::LD + k) = v[q];
      } else {
        const int k = e / (GBM / VE), r = (e % (GBM / VE)) * VE;
        const T *t = reinterpret_cast<const T *>(&v[q]);
#pragma unroll
        for (int i = 0; i < VE; i++) S[(r + i) * GemmLds<T>::LD + k] = t[i];
      }
    }
  }
};

template <typename TO>
__device__ inline void store_out(TO *p, float v);
template <>
__device__ inline void store_out<float>(float *p, float v) { *p = v; }
template <>
__device__ inline void store_out<uint16_t>(uint16_t *p, float v) { *p = f2bf(v); }

// C (or the split-K workspace slice) = A B^T over K range [kb, ke).
template <typename T, bool AKC, bool BKC, typename TO>
__global__ __launch_bounds__(256) void k_gemm(const GemmArgs g) {
  using MF = Mfma<T>;
  constexpr int LD = GemmLds<T>::LD;
  __shared__ __attribute__((aligned(16))) T sA[2][GBM * LD];
  __shared__ __attribute__((aligned(16))) T sB[2][GBN * LD];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;
  const int tiles_n = (g.N + GBN - 1) / GBN;
  const int tile = blockIdx.x, split = blockIdx.y;
  const int m0 = (tile / tiles_n) * GBM, n0 = (tile % tiles_n) * GBN;
  const int kchunk = ((g.K + g.splits - 1) / g.splits + GBK - 1) / GBK * GBK;
  const int kb = split * kchunk;
  const int ke = min(g.K, kb + kchunk);
  const T *A = (const T *)g.A, *B = (const T *)g.B;

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int j = 0; j < 2; j++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[i][j][r] = 0.f;

  TileLoader<T, AKC> la;
  TileLoader<T, BKC> lb;
  int buf = 0;
  if (kb < ke) {
    la.load(A, g.lda, g.M, ke, m0, kb, g.vec_a);
    lb.load(B, g.ldb, g.N, ke, n0, kb, g.vec_b);
    la.store(sA[0]);
    lb.store(sB[0]);
  }
  __syncthreads();
  for (int k0 = kb; k0 < ke; k0 += GBK) {
    const bool more = k0 + GBK < ke;
    if (more) {
      la.load(A, g.lda, g.M, ke, m0, k0 + GBK, g.vec_a);
      lb.load(B, g.ldb, g.N, ke, n0, k0 + GBK, g.vec_b);
    }
    const T *cA = sA[buf], *cB = sB[buf];
#pragma unroll
    for (int ks = 0; ks < GBK; ks += MF::KSTEP) {
      const int kk = ks + (lane >> 5) * MF::VEC;
#pragma unroll
      for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
          acc[i][j] = MF::mma(cA + (wm * 64 + i * 32 + (lane & 31)) * LD + kk,
                              cB + (wn * 64 + j * 32 + (lane & 31)) * LD + kk, acc[i][j]);
    }
    if (more) {
      la.store(sA[buf ^ 1]);
      lb.store(sB[buf ^ 1]);
    }
    __syncthreads();
    buf ^= 1;
  }

  // epilogue: 32x32 MFMA result, lane holds column (lane & 31) of rows
  // 8*(r/4) + 4*(lane/32) + (r%4)
  const TO *dummy = nullptr;
  (void)dummy;
#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int j = 0; j < 2; j++) {
      const int col = n0 + wn * 64 + j * 32 + (lane & 31);
      if (col >= g.N) continue;
      const float bias = (g.bias && split == 0) ? ldf((const T *)g.bias, col) : 0.f;
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int row = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row >= g.M) continue;
        const float v = acc[i][j][r] + bias;
        if (g.splits > 1) g.ws[((size_t)split * g.M + row) * g.N + col] = v;
        else store_out<TO>((TO *)g.C + (size_t)row * g.ldc + col, v);
      }
    }
}

template <typename TO>
__global__ void k_gemm_splitk_sum(const GemmArgs g) {
  const size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= (size_t)g.M * g.N) return;
  float s = 0.f;
  for (int q = 0; q < g.splits; q++) s += g.ws[(size_t)q * g.M * g.N + e];
  const size_t row = e / g.N, col = e % g.N;
  store_out<TO>((TO *)g.C + row * g.ldc + col, s);
}

template <typename T, bool AKC, bool BKC, typename TO>
static hipError_t gemm_launch(const GemmArgs &g, hipStream_t s) {
  const int tiles = ((g.M + GBM - 1) / GBM) * ((g.N + GBN - 1) / GBN);
  hipLaunchKernelGGL((k_gemm<T, AKC, BKC, TO>), dim3(tiles, g.splits), dim3(256), 0, s, g);
  if (g.splits > 1) {
    const size_t tot = (size_t)g.M * g.N;
    hipLaunchKernelGGL((k_gemm_splitk_sum<TO>), dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, s, g);
  }
  return hipGetLastError();
}

// Split K until the grid covers the device a few times over (long-K
// products such as dW = dU^T x have few output tiles), keeping at least
// 8 K tiles per split.
int gemm_splits(int M, int N, int K) {
  const int tiles = ((M + GBM - 1) / GBM) * ((N + GBN - 1) / GBN);
  int s = 1;
  while (tiles * s < 1024 && K / (s * 2) >= 8 * GBK && s < 512) s *= 2;
  return s;
}

hipError_t launch_gemm(const GemmArgs &g, hipStream_t s) {
  const bool bf = g.bf16;
#define PR_G(AKC, BKC)                                                                        \
  if (g.a_kc == AKC && g.b_kc == BKC) {                                                       \
    if (bf) return g.out_f32 ? gemm_launch<uint16_t, AKC, BKC, float>(g, s)                   \
                             : gemm_launch<uint16_t, AKC, BKC, uint16_t>(g, s);               \
    return gemm_launch<float, AKC, BKC, float>(g, s);                                         \
  }
  PR_G(true, true)
  PR_G(true, false)
  PR_G(false, true)
  PR_G(false, false)
#undef PR_G
  return hipErrorInvalidValue;
}

}  // namespace pr

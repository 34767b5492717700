// ELK with the full 64 x 64 Jacobian of the dense GRU (n = 64): the
// Levenberg-Marquardt-damped Newton step (Gonzalez et al. abstract: ELK
// stabilises DEER through the connection between Levenberg-Marquardt and
// Kalman smoothing).
//
// The damped step is the posterior mean of the linear-Gaussian model
//   dh_t = J_t dh_{t-1} + r_t + w_t,  w_t ~ N(0, I);  0 = dh_t + v_t,
//   v_t ~ N(0, I / lambda),  dh_{-1} = 0,
// which is the minimiser of
//   sum_t ||dh_t - J_t dh_{t-1} - r_t||^2 + lambda sum_t ||dh_t||^2.
// Its normal equations are block tridiagonal and symmetric positive
// definite, one 64 x 64 block row per step:
//   A_t dh_{t-1} + D_t dh_t + A_{t+1}^T dh_{t+1} = f_t,
//   A_t = -J_t,  D_t = (1 + lambda) I + J_{t+1}^T J_{t+1},
//   f_t = r_t - J_{t+1}^T r_{t+1}   (J_T = 0, r_T = 0).
// The Kalman filter with the Rauch-Tung-Striebel smoother is the sequential
// block elimination of this system (the textbook form the oracle runs); here
// the same system is eliminated in parallel over time by block cyclic
// reduction, which for an SPD system needs no pivoting.  Level s = 1, 2,
// 4, ... (while s < T) eliminates the rows j = s (2m + 1) in favour of the
// rows i = 2 s m:
//   elimination of j:  W = D_j^{-1},  P_j = W A_j,  Q_j = W A_{j+s}^T,
//                      S_j = A_j^T P_j,  g_j = W f_j,  v_j = A_j^T g_j
//   kept row i:        A_i <- -A_i P_{i-s},
//                      D_i <- D_i - A_i Q_{i-s} - S_{i+s},
//                      f_i <- f_i - A_i g_{i-s} - v_{i+s}
// (terms of a neighbour past either end drop out).  Row 0 is left: dh_0 =
// D_0^{-1} f_0; then, level by level downwards, dh_j = g_j - P_j dh_{j-s} -
// Q_j dh_{j+s}.  Every block row is eliminated once, at the cost of one SPD
// inverse (Gauss-Jordan in registers) and five 64 x 64 products on fp32 MFMA
// (v_mfma_f32_32x32x2_f32).  P_j and Q_j overwrite A_j and D_j, which the
// elimination consumes.
//
// The Jacobian's factors and the residual come from the dense GRU's gates
// kernel: J_t = diag(z) + diag(alpha) W_hz + diag(beta) W_hn + diag(gamma) W_hr.
#include <algorithm>

#include "internal.h"

namespace pr {

typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_e;

constexpr int E64_LS = 65;          // LDS row stride (floats) of a 64 x 64 matrix
constexpr int E64_MAT = 64 * E64_LS;  // floats per LDS matrix
constexpr size_t E64_NN = 4096;     // floats per stored matrix (row-major, unpadded)

// Quadrant of a 64 x 64 product held by wavefront w: rows 32 (w & 1) + ...,
// columns 32 (w >> 1) + ...; register r of lane l holds row
// 8 (r / 4) + 4 (l / 32) + r % 4 of the quadrant and column l % 32.
__device__ inline int e64_row(int r) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  return 32 * (w & 1) + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}
__device__ inline int e64_col() {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  return 32 * (w >> 1) + (lane & 31);
}

// op(X) op(Y) for 64 x 64 matrices in LDS (TX: X^T, TY: Y^T), this
// wavefront's quadrant.  256 threads.
template <bool TX, bool TY>
__device__ inline f32x16_e e64_mm(const float *X, const float *Y) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int i = 32 * (w & 1) + (lane & 31), j = 32 * (w >> 1) + (lane & 31), hl = lane >> 5;
  f32x16_e acc;
#pragma unroll
  for (int r = 0; r < 16; r++) acc[r] = 0.f;
#pragma unroll 8
  for (int s = 0; s < 32; s++) {
    const int k = 2 * s + hl;
    const float a = TX ? X[k * E64_LS + i] : X[i * E64_LS + k];
    const float b = TY ? Y[j * E64_LS + k] : Y[k * E64_LS + j];
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc, 0, 0, 0);
  }
  return acc;
}

// a stored 64 x 64 matrix (row-major, 4096 floats) into LDS
__device__ inline void e64_load(float *L, const float *G) {
  for (int e = threadIdx.x; e < 1024; e += 256) {
    const int row = e >> 4, c4 = (e & 15) * 4;
    const float4 v = *reinterpret_cast<const float4 *>(G + row * 64 + c4);
    float *d = L + row * E64_LS + c4;
    d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
  }
}
// a quadrant-layout result to global memory (row-major) or to LDS
__device__ inline void e64_store(float *G, const f32x16_e &v, float scale = 1.f) {
  const int c = e64_col();
#pragma unroll
  for (int r = 0; r < 16; r++) G[e64_row(r) * 64 + c] = scale * v[r];
}
__device__ inline void e64_put(float *L, const f32x16_e &v) {
  const int c = e64_col();
#pragma unroll
  for (int r = 0; r < 16; r++) L[e64_row(r) * E64_LS + c] = v[r];
}

// v of lane c of each quad of lanes, in every lane of the quad (c is a
// constant once the caller's loop is unrolled)
__device__ inline float e64_quad_bcast(float v, int c) {
  int x = __float_as_int(v);
  switch (c) {
    case 0: x = __builtin_amdgcn_mov_dpp(x, 0x00, 0xf, 0xf, false); break;
    case 1: x = __builtin_amdgcn_mov_dpp(x, 0x55, 0xf, 0xf, false); break;
    case 2: x = __builtin_amdgcn_mov_dpp(x, 0xaa, 0xf, 0xf, false); break;
    default: x = __builtin_amdgcn_mov_dpp(x, 0xff, 0xf, 0xf, false); break;
  }
  return __int_as_float(x);
}

// In-place inverse of an SPD 64 x 64 matrix by Gauss-Jordan elimination
// without pivoting (every pivot of an SPD matrix is positive).  Thread t
// holds row t / 4, columns 16 (t % 4) .. + 15 in m[16], so the four threads
// of a row are a quad of lanes: the pivot column's entry of a row comes from
// its owner by a quad broadcast, and only the normalised pivot row goes
// through LDS (sRow: 2 x 64 floats, double-buffered), one barrier per pivot.
__device__ inline void e64_inverse(float (&m)[16], float *sRow) {
  const int t = threadIdx.x, row = t >> 2, cq = t & 3, c0 = cq * 16;
#pragma unroll
  for (int k = 0; k < 64; k++) {
    float *R = sRow + (k & 1) * 64;
    const int kq = k >> 4, kr = k & 15;
    const float f = e64_quad_bcast(m[kr], kq);  // this row's entry in column k
    if (row == k) {  // the pivot row, divided by the pivot; 1 / pivot in column k
      const float rp = __builtin_amdgcn_rcpf(f);  // pivots of an SPD matrix: well inside the range
#pragma unroll
      for (int q = 0; q < 16; q++) R[c0 + q] = (q == kr && cq == kq) ? rp : m[q] * rp;
    }
    lds_barrier();  // orders LDS only: loads issued before the inverse stay in flight
    if (row == k) {
#pragma unroll
      for (int q = 0; q < 16; q++) m[q] = R[c0 + q];
    } else {
      if (cq == kq) m[kr] = 0.f;
#pragma unroll
      for (int q = 0; q < 16; q++) m[q] = fmaf(-f, R[c0 + q], m[q]);
    }
  }
  __syncthreads();
}

// y = M x for M held as in e64_inverse (registers) and x in LDS; returns
// y[t / 4] in every thread of the row's quad.
__device__ inline float e64_mv_regs(const float (&m)[16], const float *x) {
  const int c0 = (threadIdx.x & 3) * 16;
  float s = 0.f;
#pragma unroll
  for (int q = 0; q < 16; q++) s = fmaf(m[q], x[c0 + q], s);
  s += __shfl_xor(s, 1, 64);
  s += __shfl_xor(s, 2, 64);
  return s;
}

__device__ inline bool e64_stopped(const Elk64Args &a, int *s_stop) { return sweep_is_stopped(a.st, s_stop); }

// ---------------------------------------------------------------------------
// 1. block rows: A_t = -J_t, D_t = (1 + lambda) I + J_{t+1}^T J_{t+1},
//    f_t = r_t - J_{t+1}^T r_{t+1}; one block per run of E64_RUN steps of one
//    sequence, walked downwards so J_{t+1} is the previous step's J_t.
// ---------------------------------------------------------------------------
constexpr int E64_RUN = 16;

__global__ __launch_bounds__(256) void k_elk64_rows(const Elk64Args a) {
  __shared__ int s_stop;
  __shared__ float sW[3 * E64_MAT];  // W_hr, W_hz, W_hn
  __shared__ float sJ[E64_MAT];      // J_{t+1}, then J_t
  __shared__ float sG[256];          // z, alpha, beta, gamma of the step being built
  __shared__ float sR[2][64];        // r_{t+1} and r_t
  if (e64_stopped(a, &s_stop)) return;
  const int T = a.T, runs = (T + E64_RUN - 1) / E64_RUN;
  const int b = blockIdx.x / runs, t0 = (blockIdx.x % runs) * E64_RUN, t1 = min(T, t0 + E64_RUN);
  if (b >= a.B) return;
  for (int e = threadIdx.x; e < 192 * 16; e += 256) {
    const int row = e >> 4, c4 = (e & 15) * 4;
    const float4 v = *reinterpret_cast<const float4 *>(a.Wh + row * 64 + c4);
    float *d = sW + (row >> 6) * E64_MAT + (row & 63) * E64_LS + c4;
    d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
  }
  // J_t into sJ (and, with store, A_t = -J_t into the workspace) and r_t
  // into sR[q]; every thread calls it (it holds a barrier)
  auto build = [&](int t, int q, bool store) {
    const size_t rowi = (size_t)b * T + t;
    const float *G = a.gates + rowi * 320;
    for (int e = threadIdx.x; e < 320; e += 256) {
      if (e < 256) sG[e] = G[e];
      else sR[q][e - 256] = G[e];
    }
    __syncthreads();
    float *A = a.A + rowi * E64_NN;
    for (int e = threadIdx.x; e < 4096; e += 256) {
      const int i = e >> 6, k = e & 63;
      float v = sG[64 + i] * sW[E64_MAT + i * E64_LS + k];           // alpha W_hz
      v = fmaf(sG[128 + i], sW[2 * E64_MAT + i * E64_LS + k], v);    // beta W_hn
      v = fmaf(sG[192 + i], sW[i * E64_LS + k], v);                  // gamma W_hr
      v = i == k ? v + sG[i] : v;                                     // + diag(z)
      sJ[i * E64_LS + k] = v;
      if (store) A[e] = -v;
    }
  };
  int q = 0;  // sR buffer of r_{t+1}
  __syncthreads();  // W_h is staged
  if (t1 < T) build(t1, q, false);
  for (int t = t1 - 1; t >= t0; t--) {
    const bool nx = t + 1 < T;
    __syncthreads();  // J_{t+1} and r_{t+1} are complete
    const size_t rowi = (size_t)b * T + t;
    float *D = a.D + rowi * E64_NN;
    float fpart = 0.f;  // -(J_{t+1}^T r_{t+1})_k in thread k < 64
    if (nx) {
      const f32x16_e jj = e64_mm<true, false>(sJ, sJ);
      const int c = e64_col();
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int i = e64_row(r);
        D[i * 64 + c] = jj[r] + (i == c ? 1.f + a.lam : 0.f);
      }
      if (threadIdx.x < 64) {
        const int k = threadIdx.x;
        for (int i = 0; i < 64; i++) fpart = fmaf(-sJ[i * E64_LS + k], sR[q][i], fpart);
      }
    } else {
      for (int e = threadIdx.x; e < 4096; e += 256) D[e] = (e >> 6) == (e & 63) ? 1.f + a.lam : 0.f;
    }
    __syncthreads();  // every read of J_{t+1} is done
    build(t, q ^ 1, true);
    if (threadIdx.x < 64) a.f[rowi * 64 + threadIdx.x] = sR[q ^ 1][threadIdx.x] + fpart;  // f_t = r_t - J^T r
    q ^= 1;
  }
}

// ---------------------------------------------------------------------------
// 2. elimination of the rows j = s (2m + 1) of level s
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_elk64_elim(const Elk64Args a, int s) {
  __shared__ int s_stop;
  __shared__ float sM[2][E64_MAT];  // W (then P), A_{j+s} (then A_j)
  __shared__ float sRow[128], sV[2][64];
  if (e64_stopped(a, &s_stop)) return;
  const int T = a.T, per = (T - s + 2 * s - 1) / (2 * s);  // eliminated rows per sequence
  const int b = blockIdx.x / per, m = blockIdx.x % per, j = s * (2 * m + 1);
  if (b >= a.B || j >= T) return;
  const int t = threadIdx.x, row = t >> 2, c0 = (t & 3) * 16;
  const size_t rj = (size_t)b * T + j;
  const bool right = j + s < T;
  // D_j and A_j into registers (A_j goes to LDS once A_{j+s} is done with)
  float w[16], aj[16];
  {
    const float4 *srcD = reinterpret_cast<const float4 *>(a.D + rj * E64_NN + row * 64 + c0);
    const float4 *srcA = reinterpret_cast<const float4 *>(a.A + rj * E64_NN + row * 64 + c0);
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const float4 v = srcD[q], u = srcA[q];
      w[4 * q] = v.x; w[4 * q + 1] = v.y; w[4 * q + 2] = v.z; w[4 * q + 3] = v.w;
      aj[4 * q] = u.x; aj[4 * q + 1] = u.y; aj[4 * q + 2] = u.z; aj[4 * q + 3] = u.w;
    }
  }
  if (right) e64_load(sM[1], a.A + (rj + s) * E64_NN);
  if (t < 64) sV[0][t] = a.f[rj * 64 + t];
  e64_inverse(w, sRow);  // ends with a barrier: sM[1] and sV[0] are in
#pragma unroll
  for (int q = 0; q < 16; q++) sM[0][row * E64_LS + c0 + q] = w[q];
  const float gv = e64_mv_regs(w, sV[0]);  // g_j = W f_j
  if ((t & 3) == 0) {
    sV[1][row] = gv;
    a.g[rj * 64 + row] = gv;
  }
  __syncthreads();
  const f32x16_e Q = right ? e64_mm<false, true>(sM[0], sM[1]) : f32x16_e{};  // W A_{j+s}^T
  __syncthreads();  // every read of A_{j+s} is done
#pragma unroll
  for (int q = 0; q < 16; q++) sM[1][row * E64_LS + c0 + q] = aj[q];
  __syncthreads();
  const f32x16_e P = e64_mm<false, false>(sM[0], sM[1]);  // W A_j
  if (t < 64) {  // v_j = A_j^T g_j
    float sacc = 0.f;
    for (int i = 0; i < 64; i++) sacc = fmaf(sM[1][i * E64_LS + t], sV[1][i], sacc);
    a.v[rj * 64 + t] = sacc;
  }
  __syncthreads();  // every read of W is done
  e64_put(sM[0], P);
  __syncthreads();
  const f32x16_e S = e64_mm<true, false>(sM[1], sM[0]);  // A_j^T P_j
  e64_store(a.S + rj * E64_NN, S);
  e64_store(a.A + rj * E64_NN, P);  // P_j in place of A_j
  e64_store(a.D + rj * E64_NN, Q);  // Q_j in place of D_j (zero without a right neighbour)
}

// ---------------------------------------------------------------------------
// 3. update of the rows i = 2 s m of level s
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_elk64_keep(const Elk64Args a, int s) {
  __shared__ int s_stop;
  __shared__ float sM[2][E64_MAT];  // A_i, P_{i-s} (then Q_{i-s})
  __shared__ float sV[64];
  if (e64_stopped(a, &s_stop)) return;
  const int T = a.T, per = (T + 2 * s - 1) / (2 * s);
  const int b = blockIdx.x / per, i = 2 * s * (blockIdx.x % per);
  if (b >= a.B || i >= T) return;
  const int t = threadIdx.x, row = t >> 2, c0 = (t & 3) * 16, c = e64_col();
  const size_t ri = (size_t)b * T + i;
  const bool left = i >= s, right = i + s < T;
  float *D = a.D + ri * E64_NN, *A = a.A + ri * E64_NN;
  // this thread's share of D_i and S_{i+s} (the product's quadrant layout)
  // and of Q_{i-s} (rows of 16), loaded ahead of the products
  float dq[16], sq[16], qq[16];
  const float *Sr = a.S + (ri + (right ? s : 0)) * E64_NN;
#pragma unroll
  for (int r = 0; r < 16; r++) {
    dq[r] = D[e64_row(r) * 64 + c];
    sq[r] = right ? Sr[e64_row(r) * 64 + c] : 0.f;
  }
  f32x16_e AP{}, AQ{};
  float fl = 0.f;
  if (left) {
    const float4 *srcQ = reinterpret_cast<const float4 *>(a.D + (ri - s) * E64_NN + row * 64 + c0);
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const float4 v = srcQ[q];
      qq[4 * q] = v.x; qq[4 * q + 1] = v.y; qq[4 * q + 2] = v.z; qq[4 * q + 3] = v.w;
    }
    e64_load(sM[0], a.A + ri * E64_NN);
    e64_load(sM[1], a.A + (ri - s) * E64_NN);  // P_{i-s}
    if (t < 64) sV[t] = a.g[(ri - s) * 64 + t];
    __syncthreads();
    AP = e64_mm<false, false>(sM[0], sM[1]);
    if (t < 64) {
      for (int k = 0; k < 64; k++) fl = fmaf(sM[0][t * E64_LS + k], sV[k], fl);
    }
    __syncthreads();  // every read of P is done
#pragma unroll
    for (int q = 0; q < 16; q++) sM[1][row * E64_LS + c0 + q] = qq[q];
    __syncthreads();
    AQ = e64_mm<false, false>(sM[0], sM[1]);
  }
#pragma unroll
  for (int r = 0; r < 16; r++) {
    const int rr = e64_row(r);
    D[rr * 64 + c] = dq[r] - AQ[r] - sq[r];
    A[rr * 64 + c] = left ? -AP[r] : 0.f;
  }
  if (t < 64) a.f[ri * 64 + t] -= fl + (right ? a.v[(ri + s) * 64 + t] : 0.f);
}

// ---------------------------------------------------------------------------
// 4. row 0 of each sequence: dh_0 = D_0^{-1} f_0
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_elk64_root(const Elk64Args a) {
  __shared__ int s_stop;
  __shared__ float sRow[128], sV[64];
  if (e64_stopped(a, &s_stop)) return;
  const int b = blockIdx.x, t = threadIdx.x, row = t >> 2, c0 = (t & 3) * 16;
  const size_t r0 = (size_t)b * a.T;
  float w[16];
  const float *src = a.D + r0 * E64_NN + row * 64 + c0;
#pragma unroll
  for (int q = 0; q < 16; q++) w[q] = src[q];
  if (t < 64) sV[t] = a.f[r0 * 64 + t];
  e64_inverse(w, sRow);
  const float xv = e64_mv_regs(w, sV);
  if ((t & 3) == 0) a.x[r0 * 64 + row] = xv;
}

// ---------------------------------------------------------------------------
// 5. back-substitution of level s: dh_j = g_j - P_j dh_{j-s} - Q_j dh_{j+s}
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_elk64_back(const Elk64Args a, int s) {
  __shared__ int s_stop;
  __shared__ float sX[2][64];
  if (e64_stopped(a, &s_stop)) return;
  const int T = a.T, per = (T - s + 2 * s - 1) / (2 * s);
  const int b = blockIdx.x / per, m = blockIdx.x % per, j = s * (2 * m + 1);
  if (b >= a.B || j >= T) return;
  const int t = threadIdx.x, row = t >> 2, c0 = (t & 3) * 16;
  const size_t rj = (size_t)b * T + j;
  const bool right = j + s < T;
  if (t < 64) {
    sX[0][t] = a.x[(rj - s) * 64 + t];
    sX[1][t] = right ? a.x[(rj + s) * 64 + t] : 0.f;
  }
  __syncthreads();
  const float *P = a.A + rj * E64_NN + row * 64 + c0, *Q = a.D + rj * E64_NN + row * 64 + c0;
  float acc = 0.f;
#pragma unroll
  for (int q = 0; q < 16; q++) acc = fmaf(P[q], sX[0][c0 + q], fmaf(Q[q], sX[1][c0 + q], acc));
  acc += __shfl_xor(acc, 1, 64);
  acc += __shfl_xor(acc, 2, 64);
  if ((t & 3) == 0) a.x[rj * 64 + row] = a.g[rj * 64 + row] - acc;
}

// ---------------------------------------------------------------------------
// 6. h += dh and max |dh| into the stop rule's shards
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_elk64_apply(const Elk64Args a) {
  __shared__ int s_stop;
  __shared__ unsigned s_dmax[4];
  if (e64_stopped(a, &s_stop)) return;
  const size_t total = (size_t)a.B * a.T * 64;
  const bool first = a.k == 1;  // the iterate is h = 0 before sweep 1
  unsigned dmax = 0;
  for (size_t e = (size_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (size_t)gridDim.x * 256) {
    const float d = a.x[e];
    a.h[e] = (first ? 0.f : a.h[e]) + d;
    const unsigned u = __float_as_uint(fabsf(d));
    dmax = u > dmax ? u : dmax;
  }
  dmax = wave_max_u32(dmax);
  if ((threadIdx.x & 63) == 0) s_dmax[threadIdx.x >> 6] = dmax;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned mx = s_dmax[0];
    for (int q = 1; q < 4; q++) mx = s_dmax[q] > mx ? s_dmax[q] : mx;
    max_agent(&a.st->dslot[a.k & 3][blockIdx.x % PR_DSHARDS], mx);
  }
}

// The passes of one ELK sweep after the gates kernel.
hipError_t launch_elk64_passes(const Elk64Args &a, hipStream_t st) {
  const int B = a.B, T = a.T;
  const unsigned runs = (unsigned)((T + E64_RUN - 1) / E64_RUN);
  hipLaunchKernelGGL(k_elk64_rows, dim3(B * runs), dim3(256), 0, st, a);
  int top = 0;
  for (int s = 1; s < T; s *= 2) {
    const int pe = (T - s + 2 * s - 1) / (2 * s), pk = (T + 2 * s - 1) / (2 * s);
    hipLaunchKernelGGL(k_elk64_elim, dim3(B * pe), dim3(256), 0, st, a, s);
    hipLaunchKernelGGL(k_elk64_keep, dim3(B * pk), dim3(256), 0, st, a, s);
    top = s;
  }
  hipLaunchKernelGGL(k_elk64_root, dim3(B), dim3(256), 0, st, a);
  for (int s = top; s >= 1; s /= 2) {
    const int pe = (T - s + 2 * s - 1) / (2 * s);
    hipLaunchKernelGGL(k_elk64_back, dim3(B * pe), dim3(256), 0, st, a, s);
    if (s == 1) break;
  }
  const size_t total = (size_t)B * T * 64;
  const unsigned grid = (unsigned)std::min<size_t>((total + 255) / 256, 4096);
  hipLaunchKernelGGL(k_elk64_apply, dim3(grid), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace pr

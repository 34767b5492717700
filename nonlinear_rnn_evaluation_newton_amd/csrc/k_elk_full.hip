// ELK sweeps: the Levenberg-Marquardt-damped Newton step with the cell's own
// Jacobian, solved as a Kalman smoother with full covariance matrices
// (Gonzalez et al. abstract: ELK stabilises DEER through the connection
// between Levenberg-Marquardt and Kalman smoothing, and keeps its speed with
// parallel Kalman smoothing; Para-Seq README, Main features: ELK solver).
//
// The damped step is the posterior mean of the linear-Gaussian model
//   dh_t = J_t dh_{t-1} + r_t + w_t,  w_t ~ N(0, I);  0 = dh_t + v_t,
//   v_t ~ N(0, I / lambda),  dh_{-1} = 0.
// The Jacobian's structure splits the state into independent chains
// ("units") of N entries: each channel's (c, h) pair of the LSTM (N = 2),
// or the whole state of a small dense cell (N = n padded to 1, 2, 4 or 8).
//
// The filter runs in parallel over chunks of L steps through the
// associative filtering elements of the temporal-parallel Kalman filter
// (Sarkka and Garcia-Fernandez): a step's element is the conditional
// N(A x_{t-1} + b, C) of x_t given x_{t-1} and the step's observation, and
// the observation's likelihood exp(-x^T J x / 2 + eta^T x) in x_{t-1}; here
//   A = rho F,  b = rho r,  C = rho I,  eta = -kappa F^T r,  J = kappa F^T F,
// with F = J_t, rho = 1 / (1 + lambda), kappa = lambda / (1 + lambda).
// Elements compose associatively; a chunk's composed element maps the
// filtered moments entering the chunk to those leaving it.  Per sweep:
//   producer          J_t and r_t at the iterate, [t][unit][N*N + N]
//   k_elkf_elem       each chunk's composed element
//   k_elkf_fcarry     filtered (m, P) entering each chunk (walk over chunks)
//   k_elkf_gains      the Kalman filter through the chunk from its carry and
//                     the Rauch-Tung-Striebel gains m^s_t = G_t m^s_{t+1} + e_t,
//                     G_t = P_t J_{t+1}^T (P^-_{t+1})^{-1}, e_t = m_t - G_t m^-_{t+1};
//                     the chunk's composed reverse map
//   k_elkf_scarry     m^s entering each chunk from the right
//   k_elkf_apply      the chunk walked backwards: h += m^s, max |m^s|
// A thread owns one (unit, chunk); consecutive lanes own consecutive units,
// so every per-step access is contiguous across a wavefront.
// lambda = 0 gives rho = 1, kappa = 0: the Newton step.
#include <algorithm>

#include "k_chan_impl.h"
#include "k_time_impl.h"
#include "internal.h"

namespace pr {

// ---------------------------------------------------------------------------
// small dense matrices (row-major N x N), fully unrolled
// ---------------------------------------------------------------------------
template <int N>
__device__ inline void mm(const float *A, const float *B, float *C) {  // C = A B
#pragma unroll
  for (int i = 0; i < N; i++)
#pragma unroll
    for (int j = 0; j < N; j++) {
      float s = 0.f;
#pragma unroll
      for (int k = 0; k < N; k++) s = fmaf(A[i * N + k], B[k * N + j], s);
      C[i * N + j] = s;
    }
}
template <int N>
__device__ inline void mm_bt(const float *A, const float *B, float *C) {  // C = A B^T
#pragma unroll
  for (int i = 0; i < N; i++)
#pragma unroll
    for (int j = 0; j < N; j++) {
      float s = 0.f;
#pragma unroll
      for (int k = 0; k < N; k++) s = fmaf(A[i * N + k], B[j * N + k], s);
      C[i * N + j] = s;
    }
}
template <int N>
__device__ inline void mm_at(const float *A, const float *B, float *C) {  // C = A^T B
#pragma unroll
  for (int i = 0; i < N; i++)
#pragma unroll
    for (int j = 0; j < N; j++) {
      float s = 0.f;
#pragma unroll
      for (int k = 0; k < N; k++) s = fmaf(A[k * N + i], B[k * N + j], s);
      C[i * N + j] = s;
    }
}
template <int N>
__device__ inline void mv(const float *A, const float *x, float *y) {  // y = A x
#pragma unroll
  for (int i = 0; i < N; i++) {
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < N; k++) s = fmaf(A[i * N + k], x[k], s);
    y[i] = s;
  }
}
template <int N>
__device__ inline void mtv(const float *A, const float *x, float *y) {  // y = A^T x
#pragma unroll
  for (int i = 0; i < N; i++) {
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < N; k++) s = fmaf(A[k * N + i], x[k], s);
    y[i] = s;
  }
}
template <int N>
__device__ inline void add_identity(float *A, float s) {
#pragma unroll
  for (int i = 0; i < N; i++) A[i * N + i] += s;
}
template <int N>
__device__ inline void symmetrize(float *A) {
#pragma unroll
  for (int i = 0; i < N; i++)
#pragma unroll
    for (int j = i + 1; j < N; j++) {
      const float v = 0.5f * (A[i * N + j] + A[j * N + i]);
      A[i * N + j] = v;
      A[j * N + i] = v;
    }
}

// R = A^{-1}: closed forms for N <= 2, else Gauss-Jordan elimination with
// partial pivoting (the row exchanges are selects, so every index stays
// static and the matrix stays in registers).  The matrices inverted here
// (I + C J with C, J symmetric positive semidefinite, and covariances plus
// the identity) have eigenvalues of at least 1 in exact arithmetic.
template <int N>
__device__ inline void minv(const float *A, float *R) {
  if constexpr (N == 1) {
    R[0] = 1.f / A[0];
  } else if constexpr (N == 2) {
    const float id = 1.f / fmaf(A[0], A[3], -A[1] * A[2]);
    R[0] = A[3] * id;
    R[1] = -A[1] * id;
    R[2] = -A[2] * id;
    R[3] = A[0] * id;
  } else {
    float M[N][2 * N];
#pragma unroll
    for (int i = 0; i < N; i++)
#pragma unroll
      for (int j = 0; j < N; j++) {
        M[i][j] = A[i * N + j];
        M[i][N + j] = i == j ? 1.f : 0.f;
      }
#pragma unroll
    for (int k = 0; k < N; k++) {
#pragma unroll
      for (int r = k + 1; r < N; r++) {  // bring the largest pivot candidate to row k
        const bool sw = fabsf(M[r][k]) > fabsf(M[k][k]);
#pragma unroll
        for (int j = 0; j < 2 * N; j++) {
          const float a = M[k][j], b = M[r][j];
          M[k][j] = sw ? b : a;
          M[r][j] = sw ? a : b;
        }
      }
      const float ip = 1.f / M[k][k];
#pragma unroll
      for (int j = 0; j < 2 * N; j++) M[k][j] *= ip;
#pragma unroll
      for (int r = 0; r < N; r++) {
        if (r == k) continue;
        const float f = M[r][k];
#pragma unroll
        for (int j = 0; j < 2 * N; j++) M[r][j] = fmaf(-f, M[k][j], M[r][j]);
      }
    }
#pragma unroll
    for (int i = 0; i < N; i++)
#pragma unroll
      for (int j = 0; j < N; j++) R[i * N + j] = M[i][N + j];
  }
}

// ---------------------------------------------------------------------------
// filtering elements
// ---------------------------------------------------------------------------
template <int N>
struct Elem {
  float A[N * N], b[N], C[N * N], eta[N], J[N * N];
};
template <int N>
constexpr int elem_floats() {
  return 3 * N * N + 2 * N;
}

// the element of one step: transition F, offset r
template <int N>
__device__ inline void elem_step(const float *F, const float *r, float rho, float kap, Elem<N> &E) {
#pragma unroll
  for (int i = 0; i < N * N; i++) {
    E.A[i] = rho * F[i];
    E.C[i] = 0.f;
  }
  add_identity<N>(E.C, rho);
  float ftr[N];
  mtv<N>(F, r, ftr);
#pragma unroll
  for (int i = 0; i < N; i++) {
    E.b[i] = rho * r[i];
    E.eta[i] = -kap * ftr[i];
  }
  mm_at<N>(F, F, E.J);
#pragma unroll
  for (int i = 0; i < N * N; i++) E.J[i] *= kap;
}

// X <- X (earlier) composed with Y (later):
//   M = (I + C_x J_y)^{-1},
//   A = A_y M A_x,  b = A_y M (b_x + C_x eta_y) + b_y,  C = A_y M C_x A_y^T + C_y,
//   eta = A_x^T M^T (eta_y - J_y b_x) + eta_x,  J = A_x^T M^T J_y A_x + J_x
// ((I + J_y C_x)^{-1} = M^T since C and J are symmetric).
template <int N>
__device__ inline void elem_combine(Elem<N> &X, const Elem<N> &Y) {
  float T1[N * N], M[N * N], AM[N * N], T2[N * N];
  mm<N>(X.C, Y.J, T1);
  add_identity<N>(T1, 1.f);
  minv<N>(T1, M);
  mm<N>(Y.A, M, AM);
  // eta and J first: they need the old A_x and b_x
  float w[N], w2[N], ne[N];
  mv<N>(Y.J, X.b, w);
#pragma unroll
  for (int i = 0; i < N; i++) w[i] = Y.eta[i] - w[i];
  mtv<N>(M, w, w2);
  mtv<N>(X.A, w2, ne);
  float JA[N * N], MJA[N * N], nJ[N * N];
  mm<N>(Y.J, X.A, JA);
  mm_at<N>(M, JA, MJA);
  mm_at<N>(X.A, MJA, nJ);
  // b and C
  float t[N], nb[N];
  mv<N>(X.C, Y.eta, t);
#pragma unroll
  for (int i = 0; i < N; i++) t[i] += X.b[i];
  mv<N>(AM, t, nb);
  float nC[N * N];
  mm<N>(AM, X.C, T2);
  mm_bt<N>(T2, Y.A, nC);
  float nA[N * N];
  mm<N>(AM, X.A, nA);
#pragma unroll
  for (int i = 0; i < N; i++) {
    X.b[i] = nb[i] + Y.b[i];
    X.eta[i] = ne[i] + X.eta[i];
  }
#pragma unroll
  for (int i = 0; i < N * N; i++) {
    X.A[i] = nA[i];
    X.C[i] = nC[i] + Y.C[i];
    X.J[i] = nJ[i] + X.J[i];
  }
  symmetrize<N>(X.C);
  symmetrize<N>(X.J);
}

// filtered moments (m, P) entering a chunk -> leaving it, through the
// chunk's element E (the moments as an element with A = 0, b = m, C = P):
//   m' = A_E (I + P J_E)^{-1} (m + P eta_E) + b_E,  P' = A_E (I + P J_E)^{-1} P A_E^T + C_E
template <int N>
__device__ inline void elem_apply(const Elem<N> &E, float *m, float *P) {
  float T1[N * N], M[N * N], AM[N * N], T2[N * N], nP[N * N];
  mm<N>(P, E.J, T1);
  add_identity<N>(T1, 1.f);
  minv<N>(T1, M);
  mm<N>(E.A, M, AM);
  float t[N], nm[N];
  mv<N>(P, E.eta, t);
#pragma unroll
  for (int i = 0; i < N; i++) t[i] += m[i];
  mv<N>(AM, t, nm);
  mm<N>(AM, P, T2);
  mm_bt<N>(T2, E.A, nP);
#pragma unroll
  for (int i = 0; i < N; i++) m[i] = nm[i] + E.b[i];
#pragma unroll
  for (int i = 0; i < N * N; i++) P[i] = nP[i] + E.C[i];
  symmetrize<N>(P);
}

// ---------------------------------------------------------------------------
// geometry
// ---------------------------------------------------------------------------
struct ElkfGeom {
  int u, c, t0, t1;  // unit, chunk, the chunk's steps [t0, t1)
  bool on;
};
__device__ inline ElkfGeom elkf_geom(const ElkFullArgs &a) {
  ElkfGeom g;
  const size_t id = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  g.u = (int)(id % a.units);
  g.c = (int)(id / a.units);
  g.on = g.c < a.cpu;
  g.t0 = g.c * a.L;
  g.t1 = min(a.T, g.t0 + a.L);
  return g;
}
template <int N>
__device__ inline const float *jr_at(const ElkFullArgs &a, int t, int u) {
  return a.jr + ((size_t)t * a.units + u) * (N * N + N);
}
template <int N>
__device__ inline float *ge_at(const ElkFullArgs &a, int t, int u) {
  return a.ge + ((size_t)t * a.units + u) * (N * N + N);
}
__device__ inline size_t per_chunk(const ElkFullArgs &a, int c, int u) { return (size_t)c * a.units + u; }

template <int N>
__device__ inline void ld_jr(const ElkFullArgs &a, int t, int u, float *F, float *r) {
  const float *p = jr_at<N>(a, t, u);
#pragma unroll
  for (int i = 0; i < N * N; i++) F[i] = p[i];
#pragma unroll
  for (int i = 0; i < N; i++) r[i] = p[N * N + i];
}

// ---------------------------------------------------------------------------
// producers: J_t and r_t at the iterate (they open the sweep)
// ---------------------------------------------------------------------------
// LSTM: one thread per (sequence, step, channel); unit = b * n + c.
template <typename ST>
__global__ __launch_bounds__(256) void k_elkf_jr_lstm(const ElkFullArgs a) {
  __shared__ int s_stop;
  if (sweep_open(a.st, a.k, a.tol, a.T, a.max_iters, &s_stop)) return;
  const int n = a.n, T = a.T, S = 2 * n;
  const bool first = a.k == 1;  // the iterate is h = 0 before sweep 1
  const size_t total = (size_t)a.B * T * n;
  const ST *U = (const ST *)a.U, *h = (const ST *)a.h, *h0 = (const ST *)a.h0;
  const ST *Wh = (const ST *)a.Wh, *bh = (const ST *)a.bh, *pe = (const ST *)a.peep;
  for (size_t id = (size_t)blockIdx.x * blockDim.x + threadIdx.x; id < total; id += (size_t)gridDim.x * blockDim.x) {
    const int c = (int)(id % n);
    const size_t row = id / n;  // b * T + t
    const int t = (int)(row % T), b = (int)(row / T);
    ChanW w;
    w.a0 = ldf(Wh, c); w.a1 = ldf(Wh, (size_t)n + c); w.a2 = ldf(Wh, (size_t)2 * n + c);
    w.b0 = bh ? ldf(bh, c) : 0.f; w.b1 = bh ? ldf(bh, (size_t)n + c) : 0.f; w.b2 = bh ? ldf(bh, (size_t)2 * n + c) : 0.f;
    w.p0 = ldf(pe, c); w.p1 = ldf(pe, (size_t)n + c);
    chan_w_scale<C_LSTM>(w);
    float u[3], s[2], hc[2], f[2], J[4];
#pragma unroll
    for (int q = 0; q < 3; q++) u[q] = ldf(U, row * 3 * n + (size_t)q * n + c);
#pragma unroll
    for (int q = 0; q < 2; q++) {
      if (t > 0) s[q] = first ? 0.f : ldf(h, (row - 1) * S + 2 * c + q);
      else s[q] = h0 ? ldf(h0, (size_t)b * S + 2 * c + q) : 0.f;
      hc[q] = first ? 0.f : ldf(h, row * S + 2 * c + q);
    }
    chan_cell<C_LSTM>(s, u, w, f, J);
    float *o = a.jr + ((size_t)t * a.units + (size_t)b * n + c) * 6;
#pragma unroll
    for (int q = 0; q < 4; q++) o[q] = J[q];
    o[4] = f[0] - hc[0];
    o[5] = f[1] - hc[1];
  }
}

// small dense cells: one thread per (sequence, step); unit = b; the padded
// rows and columns of J and entries of r are zero.
template <int N, int CELL, int DX>
__global__ __launch_bounds__(256) void k_elkf_jr_dense(const TimeArgs ta, const ElkFullArgs a) {
  constexpr int G = cell_gates(CELL);
  __shared__ float sWh[G * N * N], sbh[G * N], sWx[G * N * DX], sbx[G * N];
  __shared__ int s_stop;
  if (sweep_open(a.st, a.k, a.tol, a.T, a.max_iters, &s_stop)) return;
  stage_dense_weights<N, G, DX>(ta, sWh, sbh, sWx, sbx);
  __syncthreads();
  const int n = ta.n, d = ta.d, T = ta.T;
  const size_t rows = (size_t)ta.B * T;
  const bool first = a.k == 1;
  for (size_t row = (size_t)blockIdx.x * blockDim.x + threadIdx.x; row < rows; row += (size_t)gridDim.x * blockDim.x) {
    const int t = (int)(row % T), b = (int)(row / T);
    float xt[DX], sp[N], hc[N], U[G * N], f[N], J[N * N];
#pragma unroll
    for (int c = 0; c < DX; c++) xt[c] = c < d ? ta.x[row * d + c] : 0.f;
#pragma unroll
    for (int i = 0; i < N; i++) {
      float v = 0.f;
      if (i < n) {
        if (t > 0) v = first ? 0.f : ta.h[(row - 1) * n + i];
        else if (ta.h0) v = ta.h0[(size_t)b * n + i];
      }
      sp[i] = v;
      hc[i] = (i < n && !first) ? ta.h[row * n + i] : 0.f;
    }
    input_proj<N, G, DX>(sWx, sbx, xt, U);
    dense_cell<N, CELL>(sp, U, sWh, sbh, f, J);
    float *o = a.jr + ((size_t)t * a.units + b) * (N * N + N);
#pragma unroll
    for (int i = 0; i < N; i++) {
#pragma unroll
      for (int j = 0; j < N; j++) o[i * N + j] = (i < n && j < n) ? J[i * N + j] : 0.f;
      o[N * N + i] = i < n ? f[i] - hc[i] : 0.f;
    }
  }
}

// ---------------------------------------------------------------------------
// 1. each chunk's composed filtering element
// ---------------------------------------------------------------------------
template <int N>
__global__ __launch_bounds__(256) void k_elkf_elem(const ElkFullArgs a) {
  __shared__ int s_stop;
  if (sweep_is_stopped(a.st, &s_stop)) return;
  const ElkfGeom g = elkf_geom(a);
  if (!g.on) return;
  const float rho = 1.f / (1.f + a.lam), kap = a.lam * rho;
  Elem<N> E, Y;
  float F[N * N], r[N];
  ld_jr<N>(a, g.t0, g.u, F, r);
  elem_step<N>(F, r, rho, kap, E);
  for (int t = g.t0 + 1; t < g.t1; t++) {
    ld_jr<N>(a, t, g.u, F, r);
    elem_step<N>(F, r, rho, kap, Y);
    elem_combine<N>(E, Y);
  }
  float *o = a.elem + per_chunk(a, g.c, g.u) * elem_floats<N>();
#pragma unroll
  for (int i = 0; i < N * N; i++) {
    o[i] = E.A[i];
    o[N * N + N + i] = E.C[i];
    o[2 * N * N + 2 * N + i] = E.J[i];
  }
#pragma unroll
  for (int i = 0; i < N; i++) {
    o[N * N + i] = E.b[i];
    o[2 * N * N + N + i] = E.eta[i];
  }
}

template <int N>
__device__ inline void ld_elem(const float *p, Elem<N> &E) {
#pragma unroll
  for (int i = 0; i < N * N; i++) {
    E.A[i] = p[i];
    E.C[i] = p[N * N + N + i];
    E.J[i] = p[2 * N * N + 2 * N + i];
  }
#pragma unroll
  for (int i = 0; i < N; i++) {
    E.b[i] = p[N * N + i];
    E.eta[i] = p[2 * N * N + N + i];
  }
}

// ---------------------------------------------------------------------------
// 2. filtered (m, P) entering each chunk: one thread per unit walks its chunks
// (the next chunk's element is loaded while the current one is applied)
// ---------------------------------------------------------------------------
template <int N>
__global__ __launch_bounds__(64) void k_elkf_fcarry(const ElkFullArgs a) {
  __shared__ int s_stop;
  if (sweep_is_stopped(a.st, &s_stop)) return;
  const int u = blockIdx.x * blockDim.x + threadIdx.x;
  if (u >= a.units) return;
  float m[N], P[N * N];
#pragma unroll
  for (int i = 0; i < N; i++) m[i] = 0.f;
#pragma unroll
  for (int i = 0; i < N * N; i++) P[i] = 0.f;
  Elem<N> E[2];
  ld_elem<N>(a.elem + per_chunk(a, 0, u) * elem_floats<N>(), E[0]);
  for (int c = 0; c < a.cpu; c++) {
    if (c + 1 < a.cpu) ld_elem<N>(a.elem + per_chunk(a, c + 1, u) * elem_floats<N>(), E[(c + 1) & 1]);
    float *o = a.fin + per_chunk(a, c, u) * (N + N * N);
#pragma unroll
    for (int i = 0; i < N; i++) o[i] = m[i];
#pragma unroll
    for (int i = 0; i < N * N; i++) o[N + i] = P[i];
    elem_apply<N>(E[c & 1], m, P);
  }
}

// ---------------------------------------------------------------------------
// 3. the filter through each chunk from its carry; smoother gains G_t, e_t per
// step and the chunk's reverse map m^s_{t0} = Mr m^s_{t1} + vr
// ---------------------------------------------------------------------------
template <int N>
__device__ inline void kf_predict(const float *F, const float *r, const float *m, const float *P, float *mp, float *Pp) {
  float FP[N * N];
  mm<N>(F, P, FP);
  mm_bt<N>(FP, F, Pp);
  add_identity<N>(Pp, 1.f);
  symmetrize<N>(Pp);
  mv<N>(F, m, mp);
#pragma unroll
  for (int i = 0; i < N; i++) mp[i] += r[i];
}

template <int N>
__global__ __launch_bounds__(256) void k_elkf_gains(const ElkFullArgs a) {
  __shared__ int s_stop;
  if (sweep_is_stopped(a.st, &s_stop)) return;
  const ElkfGeom g = elkf_geom(a);
  if (!g.on) return;
  float m[N], P[N * N], Mr[N * N], vr[N];
  {
    const float *in = a.fin + per_chunk(a, g.c, g.u) * (N + N * N);
#pragma unroll
    for (int i = 0; i < N; i++) {
      m[i] = in[i];
      vr[i] = 0.f;
    }
#pragma unroll
    for (int i = 0; i < N * N; i++) {
      P[i] = in[N + i];
      Mr[i] = 0.f;
    }
    add_identity<N>(Mr, 1.f);
  }
  const int tend = g.t1 < a.T ? g.t1 + 1 : g.t1;  // one step into the next chunk for the last gain
  for (int t = g.t0; t < tend; t++) {
    float F[N * N], r[N], mp[N], Pp[N * N];
    ld_jr<N>(a, t, g.u, F, r);
    kf_predict<N>(F, r, m, P, mp, Pp);
    if (t > g.t0) {  // the gain of step t - 1: G = P_{t-1} F^T (P^-_t)^{-1}, e = m_{t-1} - G m^-_t
      float Pi[N * N], PF[N * N], G[N * N], e[N];
      minv<N>(Pp, Pi);
      mm_bt<N>(P, F, PF);
      mm<N>(PF, Pi, G);
      mv<N>(G, mp, e);
#pragma unroll
      for (int i = 0; i < N; i++) e[i] = m[i] - e[i];
      float *o = ge_at<N>(a, t - 1, g.u);
#pragma unroll
      for (int i = 0; i < N * N; i++) o[i] = G[i];
#pragma unroll
      for (int i = 0; i < N; i++) o[N * N + i] = e[i];
      // m^s_{t0} = Mr m^s_{t-1} + vr and m^s_{t-1} = G m^s_t + e
      float Me[N], MG[N * N];
      mv<N>(Mr, e, Me);
      mm<N>(Mr, G, MG);
#pragma unroll
      for (int i = 0; i < N; i++) vr[i] += Me[i];
#pragma unroll
      for (int i = 0; i < N * N; i++) Mr[i] = MG[i];
    }
    if (t == g.t1) break;  // the next chunk's first step only served the last gain
    // update: P = (lambda P^- + I)^{-1} P^-, m = (lambda P^- + I)^{-1} m^-
    float Aq[N * N], Ai[N * N];
#pragma unroll
    for (int i = 0; i < N * N; i++) Aq[i] = a.lam * Pp[i];
    add_identity<N>(Aq, 1.f);
    minv<N>(Aq, Ai);
    mm<N>(Ai, Pp, P);
    symmetrize<N>(P);
    mv<N>(Ai, mp, m);
  }
  if (g.t1 == a.T) {  // the sequence's last step: m^s = m, G = 0
    float *o = ge_at<N>(a, a.T - 1, g.u);
#pragma unroll
    for (int i = 0; i < N * N; i++) o[i] = 0.f;
#pragma unroll
    for (int i = 0; i < N; i++) o[N * N + i] = m[i];
    float Me[N];
    mv<N>(Mr, m, Me);
#pragma unroll
    for (int i = 0; i < N; i++) vr[i] += Me[i];
#pragma unroll
    for (int i = 0; i < N * N; i++) Mr[i] = 0.f;
  }
  float *o = a.rev + per_chunk(a, g.c, g.u) * (N * N + N);
#pragma unroll
  for (int i = 0; i < N * N; i++) o[i] = Mr[i];
#pragma unroll
  for (int i = 0; i < N; i++) o[N * N + i] = vr[i];
}

// ---------------------------------------------------------------------------
// 4. m^s entering each chunk from the right: one thread per unit
// ---------------------------------------------------------------------------
template <int N>
__global__ __launch_bounds__(64) void k_elkf_scarry(const ElkFullArgs a) {
  __shared__ int s_stop;
  if (sweep_is_stopped(a.st, &s_stop)) return;
  const int u = blockIdx.x * blockDim.x + threadIdx.x;
  if (u >= a.units) return;
  float x[N];
#pragma unroll
  for (int i = 0; i < N; i++) x[i] = 0.f;
  float R[2][N * N + N];
  auto load = [&](int c, float *dst) {
    const float *p = a.rev + per_chunk(a, c, u) * (N * N + N);
#pragma unroll
    for (int i = 0; i < N * N + N; i++) dst[i] = p[i];
  };
  load(a.cpu - 1, R[(a.cpu - 1) & 1]);
  for (int c = a.cpu - 1; c >= 0; c--) {
    if (c > 0) load(c - 1, R[(c - 1) & 1]);
    float *o = a.msin + per_chunk(a, c, u) * N;
#pragma unroll
    for (int i = 0; i < N; i++) o[i] = x[i];
    const float *Rc = R[c & 1];
    float y[N];
    mv<N>(Rc, x, y);
#pragma unroll
    for (int i = 0; i < N; i++) x[i] = y[i] + Rc[N * N + i];
  }
}

// ---------------------------------------------------------------------------
// 5. each chunk walked backwards from its right-hand carry: h += m^s, max |m^s|
// ---------------------------------------------------------------------------
template <int N, typename ST>
__global__ __launch_bounds__(256) void k_elkf_apply(const ElkFullArgs a) {
  __shared__ int s_stop;
  __shared__ unsigned s_dmax[4];
  if (sweep_is_stopped(a.st, &s_stop)) return;
  const ElkfGeom g = elkf_geom(a);
  const bool first = a.k == 1;  // the iterate is h = 0 before sweep 1
  unsigned dmax = 0;
  if (g.on) {
    float y[N];
    const float *in = a.msin + per_chunk(a, g.c, g.u) * N;
#pragma unroll
    for (int i = 0; i < N; i++) y[i] = in[i];
    ST *h = (ST *)a.h;
    const int b = g.u / a.upb, cu = g.u % a.upb;
    for (int t = g.t1 - 1; t >= g.t0; t--) {
      const float *p = ge_at<N>(a, t, g.u);
      float ny[N];
#pragma unroll
      for (int i = 0; i < N; i++) {
        float s = p[N * N + i];
#pragma unroll
        for (int k = 0; k < N; k++) s = fmaf(p[i * N + k], y[k], s);
        ny[i] = s;
      }
      const size_t base = ((size_t)b * a.T + t) * a.S + (size_t)cu * a.NS;
#pragma unroll
      for (int i = 0; i < N; i++) {
        y[i] = ny[i];
        if (i < a.NS) {
          const float hv = first ? 0.f : ldf(h, base + i);
          stf(h, base + i, hv + y[i]);
          const unsigned uv = __float_as_uint(fabsf(y[i]));
          dmax = uv > dmax ? uv : dmax;
        }
      }
    }
  }
  dmax = wave_max_u32(dmax);
  if ((threadIdx.x & 63) == 0) s_dmax[threadIdx.x >> 6] = dmax;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned mx = s_dmax[0];
    for (int q = 1; q < (int)(blockDim.x >> 6); q++) mx = s_dmax[q] > mx ? s_dmax[q] : mx;
    max_agent(&a.st->dslot[a.k & 3][blockIdx.x % PR_DSHARDS], mx);
  }
}

// ---------------------------------------------------------------------------
// launch
// ---------------------------------------------------------------------------
// Steps per chunk: about sqrt(T) (the chunk passes walk L steps, the carries
// T / L chunks), at least 8, and at most 256 chunks per unit.
int elk_full_chunk_len(int T) {
  int L = 8;
  while (L * L < T) L *= 2;
  while ((T + L - 1) / L > 256) L *= 2;
  return L;
}

template <int N, typename ST>
static hipError_t elkf_passes(const ElkFullArgs &a, hipStream_t s) {
  const size_t threads = (size_t)a.units * a.cpu;
  const unsigned gpc = (unsigned)((threads + 255) / 256);
  const unsigned gpu = (unsigned)((a.units + 63) / 64);
  hipLaunchKernelGGL((k_elkf_elem<N>), dim3(gpc), dim3(256), 0, s, a);
  hipLaunchKernelGGL((k_elkf_fcarry<N>), dim3(gpu), dim3(64), 0, s, a);
  hipLaunchKernelGGL((k_elkf_gains<N>), dim3(gpc), dim3(256), 0, s, a);
  hipLaunchKernelGGL((k_elkf_scarry<N>), dim3(gpu), dim3(64), 0, s, a);
  hipLaunchKernelGGL((k_elkf_apply<N, ST>), dim3(gpc), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_elk_full_lstm(bool bf16, const ElkFullArgs &a, hipStream_t s) {
  const size_t total = (size_t)a.B * a.T * a.n;
  const unsigned grid = (unsigned)std::min<size_t>((total + 255) / 256, 1u << 20);
  if (bf16) hipLaunchKernelGGL((k_elkf_jr_lstm<uint16_t>), dim3(grid), dim3(256), 0, s, a);
  else hipLaunchKernelGGL((k_elkf_jr_lstm<float>), dim3(grid), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return bf16 ? elkf_passes<2, uint16_t>(a, s) : elkf_passes<2, float>(a, s);
}

template <int CELL>
static hipError_t elkf_dense_cell(int Nv, const TimeArgs &ta, const ElkFullArgs &a, hipStream_t s) {
  const size_t rows = (size_t)ta.B * ta.T;
  const unsigned grid = (unsigned)std::min<size_t>((rows + 255) / 256, 65536);
  PR_DISPATCH_N(Nv, PR_DISPATCH_DX(ta.d, {
    hipLaunchKernelGGL((k_elkf_jr_dense<N, CELL, DX>), dim3(grid), dim3(256), 0, s, ta, a);
  }));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  switch (Nv) {
    case 1: return elkf_passes<1, float>(a, s);
    case 2: return elkf_passes<2, float>(a, s);
    case 4: return elkf_passes<4, float>(a, s);
    case 8: return elkf_passes<8, float>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_elk_full_dense(int cell, int Nv, const TimeArgs &ta, const ElkFullArgs &a, hipStream_t s) {
  switch (cell) {
    case C_TANH: return elkf_dense_cell<C_TANH>(Nv, ta, a, s);
    case C_GRU: return elkf_dense_cell<C_GRU>(Nv, ta, a, s);
    case C_LINEAR: return elkf_dense_cell<C_LINEAR>(Nv, ta, a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace pr

// Linear state-space simulation (the Para-Seq README's lsim, Main features:
// ODE solvers; Example: lsim(A, B, C, D, U, t)) through the same kind of
// affine scan the Newton sweeps use, with no Newton loop: the system
// dx/dt = A x + B u, y = C x + D u is sampled on uniform times with the
// input held between samples (zero-order hold), so
//   x_0 = x0,  y_k = C x_k + D u_k,  x_{k+1} = Ad x_k + Bd u_k,
//   Ad = exp(A dt),  Bd = int_0^dt exp(A s) ds B.
// The operator Ad is the same at every step, so a scan only carries vectors:
// composing a run of n steps multiplies by Ad^n, taken from a table of
// powers.  A lane owns V consecutive steps, a wavefront a chunk of 64 V.
// Four launches:
//  1. k_lsim_disc (one wavefront): Ad, Bd from one fp64 matrix exponential
//     of the augmented matrix [[A, B], [0, 0]] dt (scaling and squaring with
//     a Taylor polynomial), and the tables (Ad^V)^(2^i) and P^(2^i),
//     P = Ad^(64 V);
//  2. k_lsim_pass<false>: each lane composes its V steps from the zero
//     state, a wavefront scan (offsets 1..32, multiplier (Ad^V)^offset)
//     composes the chunk; its state from 0 is the chunk's aggregate;
//  3. k_lsim_carry: one wavefront per sequence, lane = chunk: the same scan
//     over chunk aggregates with multipliers P^offset gives each chunk's
//     entering state;
//  4. k_lsim_pass<true>: the chunk again from its entering state; each lane
//     replays its V steps, storing x_k and y_k.
#include "internal.h"

namespace pr {

constexpr int LS_W = 8;                 // largest state, input and output width
constexpr int LS_MAT = LS_W * LS_W;     // floats per (padded) matrix
constexpr int LS_R = 16;                // rounds of 64 V steps per chunk (a power of two)
constexpr int LS_LOGR = 4;
constexpr int LS_PW = 6 + LS_LOGR;      // powers P^(2^i) kept, P = Ad^(64 V)
constexpr int LS_TABLE = 2 + 6 + LS_PW; // Ad, Bd, (Ad^V)^(2^i) i < 6, P^(2^i) i < LS_PW

// steps per lane in a round (short runs keep the output staging small, so
// many wavefronts fit on a CU)
constexpr int ls_v(int) { return 4; }
static int ls_mpad(int m) { return m <= 1 ? 1 : m <= 2 ? 2 : m <= 4 ? 4 : 8; }

// workspace floats before the chunk arrays
int lsim_table_floats() { return LS_TABLE * LS_MAT; }
int lsim_chunk_len(int m) { return 64 * LS_R * ls_v(ls_mpad(m)); }

// Ordering of LDS accesses within one wavefront: its LDS writes are visible
// to its later reads once they have completed, so a wait on the LDS counter
// alone orders them (a memory fence would also wait for the wavefront's
// outstanding global stores).
__device__ inline void ls_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_wave_barrier();
}

// C = A B for S x S row-major fp64 matrices in LDS (zero padded; each lane
// takes S * S / 64 entries, all their LDS reads in flight together)
template <int LS_S>
__device__ inline void ls_matmul(const double *A, const double *B, double *C) {
  const int lane = threadIdx.x;
#pragma unroll
  for (int q = 0; q < LS_S * LS_S / 64; q++) {
    const int e = lane + 64 * q, i = e / LS_S, j = e % LS_S;
    double s = 0.0;
#pragma unroll
    for (int k = 0; k < LS_S; k++) s = fma(A[i * LS_S + k], B[k * LS_S + j], s);
    C[e] = s;
  }
  ls_sync();
}

// M <- M M (through Tm)
template <int LS_S>
__device__ inline void ls_square(double *M, double *Tm) {
  ls_matmul<LS_S>(M, M, Tm);
#pragma unroll
  for (int q = 0; q < LS_S * LS_S / 64; q++) M[threadIdx.x + 64 * q] = Tm[threadIdx.x + 64 * q];
  ls_sync();
}

// padded fp32 copy of the r x c block of M at column c0
template <int LS_S>
__device__ inline void ls_store(const double *M, int r, int c, int c0, float *out) {
  const int e = threadIdx.x, i = e / LS_W, j = e % LS_W;  // LS_MAT = 64 entries, one per lane
  out[e] = (i < r && j < c) ? (float)M[i * LS_S + c0 + j] : 0.f;
}

// LS_S: the augmented matrix's size nx + m padded to 8 or 16
template <int LS_S>
__global__ __launch_bounds__(64) void k_lsim_disc(const LsimArgs a) {
  __shared__ double M[LS_S * LS_S], E[LS_S * LS_S], Tm[LS_S * LS_S];
  __shared__ int s_sq;
  const int nx = a.nx, m = a.m, n = nx + m, tid = threadIdx.x;
  // M = [[A, B], [0, 0]] dt, zero padded, and its 1-norm
#pragma unroll
  for (int q = 0; q < LS_S * LS_S / 64; q++) {
    const int e = tid + 64 * q, i = e / LS_S, j = e % LS_S;
    double v = 0.0;
    if (i < nx && j < n) v = j < nx ? (double)a.A[i * nx + j] : (double)a.Bm[i * m + (j - nx)];
    M[e] = v * (double)a.dt;
  }
  ls_sync();
  if (tid == 0) {
    double nrm = 0.0;
    for (int j = 0; j < n; j++) {
      double c = 0.0;
      for (int i = 0; i < n; i++) c += fabs(M[i * LS_S + j]);
      nrm = c > nrm ? c : nrm;
    }
    int sq = 0;
    while (nrm > 0.5 && sq < 60) {
      nrm *= 0.5;
      sq++;
    }
    s_sq = sq;
  }
  ls_sync();
  const int sq = s_sq;
  const double scale = ldexp(1.0, -sq);
#pragma unroll
  for (int q = 0; q < LS_S * LS_S / 64; q++) {
    const int e = tid + 64 * q;
    M[e] *= scale;
    E[e] = (e / LS_S == e % LS_S) ? 1.0 : 0.0;
  }
  ls_sync();
  // exp(M) ~ I + M (I + M/2 (I + M/3 (... (I + M/12)))) by Horner; with
  // ||M|| <= 1/2 the truncation is below 0.5^13 / 13! ~ 2e-14
  for (int q = 12; q >= 1; q--) {
    ls_matmul<LS_S>(M, E, Tm);
#pragma unroll
    for (int r = 0; r < LS_S * LS_S / 64; r++) {
      const int e = tid + 64 * r;
      E[e] = ((e / LS_S == e % LS_S) ? 1.0 : 0.0) + Tm[e] / (double)q;
    }
    ls_sync();
  }
  for (int r = 0; r < sq; r++) ls_square<LS_S>(E, Tm);
  float *tab = a.table;
  ls_store<LS_S>(E, nx, nx, 0, tab);           // Ad
  ls_store<LS_S>(E, nx, m, nx, tab + LS_MAT);  // Bd
  // Ad alone (zero padded), squared to Ad^V, then its powers of two up to
  // P = (Ad^V)^64, then P's
#pragma unroll
  for (int q = 0; q < LS_S * LS_S / 64; q++) {
    const int e = tid + 64 * q, i = e / LS_S, j = e % LS_S;
    M[e] = (i < nx && j < nx) ? E[e] : 0.0;
  }
  ls_sync();
  for (int v = 1; v < a.V; v *= 2) ls_square<LS_S>(M, Tm);
  for (int i = 0; i < 6 + LS_PW; i++) {  // (Ad^V)^(2^i), i < 6, then P^(2^(i - 6))
    ls_store<LS_S>(M, nx, nx, 0, tab + (2 + i) * LS_MAT);
    ls_square<LS_S>(M, Tm);
  }
}

// y = M v for a padded NX x NX matrix in LDS
template <int NX>
__device__ inline void ls_mv(const float *M, const float *v, float *y) {
#pragma unroll
  for (int i = 0; i < NX; i++) {
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < NX; j++) s = fmaf(M[i * LS_W + j], v[j], s);
    y[i] = s;
  }
}

// Inclusive wavefront scan of the vectors e (lane order = time order) under
// the maps v -> pw[i] v for offsets 2^i: afterwards lane l holds
// sum_{j <= l} Ad^(l - j) e_j (with the table of Ad^(2^i)).
template <int NX>
__device__ inline void ls_wave_scan(const float *pw, float *e) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < 6; i++) {
    const int off = 1 << i;
    float t[NX], u[NX];
#pragma unroll
    for (int r = 0; r < NX; r++) t[r] = __shfl_up(e[r], off, 64);
    ls_mv<NX>(pw + i * LS_MAT, t, u);
    if (lane >= off) {
#pragma unroll
      for (int r = 0; r < NX; r++) e[r] += u[r];
    }
  }
}

// One wavefront per chunk (b, j) of 64 V steps, lane l owning steps
// 64 V j + V l + [0, V).  APPLY = false: the chunk's state after its last step
// from the zero state (its aggregate); APPLY = true: x_k and y_k of every step
// from the chunk's entering state.  NX, MP: state and input widths padded to
// a power of two.  Only a sequence's last chunk can be partial; there every
// lane before the one holding the last step is full, so the scan's constant
// multipliers hold for every entering state that is used.
// LDS staging of a wavefront's outputs (APPLY, dynamic shared memory): rows
// [0, 64 V) of x (NX floats) and of y (p floats), one float of padding after
// each lane's V rows so the lane-strided writes hit distinct banks.
static size_t ls_stage_bytes(int NX, int V, int p) { return ((size_t)64 * V * (NX + p) + 2 * 64) * 4; }

template <int NX, int MP, bool APPLY>
__global__ __launch_bounds__(64) void k_lsim_pass(const LsimArgs a) {
  constexpr int V = ls_v(MP);
  extern __shared__ float stage[];
  // Ad, Bd, (Ad^V)^(2^i) and C, D in LDS (broadcast reads; read from global
  // memory they would be vector loads, as the outputs may alias them)
  __shared__ float tab[8 * LS_MAT], sC[LS_MAT], sD[LS_MAT];
  const int lane = threadIdx.x, chunk = blockIdx.x;
  const int T = a.T, m = a.m, p = a.p, nx = a.nx;
  for (int e = lane; e < 8 * LS_MAT; e += 64) tab[e] = a.table[e];
  if (APPLY) {
    const int i = lane / LS_W, c = lane % LS_W;
    sC[lane] = (i < p && c < nx) ? a.Cm[i * nx + c] : 0.f;
    sD[lane] = (i < p && c < m) ? a.Dm[i * m + c] : 0.f;
  }
  ls_sync();
  const int b = chunk / a.cps, j = chunk % a.cps;
  const float *pw = tab + 2 * LS_MAT;
  // the per-step operators Ad (NX x NX) and Bd (NX x MP) in registers
  float Ad[LS_MAT], Bd[LS_MAT];
#pragma unroll
  for (int r = 0; r < NX; r++) {
#pragma unroll
    for (int c = 0; c < NX; c++) Ad[r * LS_W + c] = tab[r * LS_W + c];
#pragma unroll
    for (int c = 0; c < MP; c++) Bd[r * LS_W + c] = tab[LS_MAT + r * LS_W + c];
  }
  const size_t rowb = (size_t)b * T;
  const int kc = j * LS_R * 64 * V;  // the chunk's first step
  // a lane's inputs in a round starting at k0 (addresses clamped into the
  // round, so the loads are unconditional; entries past m or T are zeroed)
  auto load = [&](int k0, float (&u)[V][MP]) __attribute__((always_inline)) {
    const int k_end = min(T, k0 + 64 * V), kl = k0 + lane * V;
#pragma unroll
    for (int v = 0; v < V; v++) {
      const size_t row = rowb + min(kl + v, k_end - 1);
#pragma unroll
      for (int c = 0; c < MP; c++) u[v][c] = a.U[row * m + min(c, m - 1)];
    }
#pragma unroll
    for (int v = 0; v < V; v++)
#pragma unroll
      for (int c = 0; c < MP; c++) u[v][c] = (c < m && kl + v < k_end) ? u[v][c] : 0.f;
  };
  float st[NX];  // state entering the round (the same in every lane)
#pragma unroll
  for (int r = 0; r < NX; r++) st[r] = (APPLY && r < nx) ? a.carry[(size_t)chunk * LS_W + r] : 0.f;
  float un[V][MP];
  load(kc, un);
  for (int rd = 0; rd < LS_R; rd++) {
    const int k0 = kc + rd * 64 * V;
    if (k0 >= T) break;
    const int k_end = min(T, k0 + 64 * V), kl = k0 + lane * V;
    float u[V][MP];
#pragma unroll
    for (int v = 0; v < V; v++)
#pragma unroll
      for (int c = 0; c < MP; c++) u[v][c] = un[v][c];
    load(k0 + 64 * V < T && rd + 1 < LS_R ? k0 + 64 * V : k0, un);  // the next round's inputs
    // the lane's V steps from the zero state
    float z[NX];
#pragma unroll
    for (int r = 0; r < NX; r++) z[r] = 0.f;
#pragma unroll
    for (int v = 0; v < V; v++) {
      float t[NX];
      ls_mv<NX>(Ad, z, t);
#pragma unroll
      for (int r = 0; r < NX; r++) {
        float s = t[r];
#pragma unroll
        for (int c = 0; c < MP; c++) s = fmaf(Bd[r * LS_W + c], u[v][c], s);
        z[r] = s;
      }
    }
    if (lane == 0) {
      float t[NX];
      ls_mv<NX>(pw, st, t);  // (Ad^V) st
#pragma unroll
      for (int r = 0; r < NX; r++) z[r] += t[r];
    }
    ls_wave_scan<NX>(pw, z);  // z = state after the lane's last step
    if constexpr (APPLY) {
      float x[NX];  // state entering the lane's first step
#pragma unroll
      for (int r = 0; r < NX; r++) {
        const float prev = __shfl_up(z[r], 1, 64);
        x[r] = lane == 0 ? st[r] : prev;
      }
      float *sx = stage, *sy = stage + 64 * V * NX + 64;
#pragma unroll
      for (int v = 0; v < V; v++) {
        const int rl = lane * V + v;  // row within the round
#pragma unroll
        for (int r = 0; r < NX; r++) sx[rl * NX + r + lane] = x[r];
        for (int o = 0; o < p; o++) {
          float s = 0.f;
#pragma unroll
          for (int r = 0; r < NX; r++) s = fmaf(sC[o * LS_W + r], x[r], s);
#pragma unroll
          for (int c = 0; c < MP; c++) s = fmaf(sD[o * LS_W + c], u[v][c], s);
          sy[rl * p + o + lane] = s;
        }
        float t[NX];
        ls_mv<NX>(Ad, x, t);
#pragma unroll
        for (int r = 0; r < NX; r++) {
          float s = t[r];
#pragma unroll
          for (int c = 0; c < MP; c++) s = fmaf(Bd[r * LS_W + c], u[v][c], s);
          x[r] = s;
        }
      }
      ls_sync();
      // coalesced copy-out of the round's rows [k0, k_end); (row, column) of
      // element e = lane + 64 i are stepped without divisions
      const int rows = k_end - k0;
      if (a.x) {
        float *gx = a.x + (rowb + k0) * nx;
        int rl = lane / nx, r = lane % nx;
        const int drl = 64 / nx, dr = 64 % nx;
        for (int e = lane; e < rows * nx; e += 64) {
          gx[e] = sx[rl * NX + r + rl / V];
          rl += drl;
          r += dr;
          if (r >= nx) { r -= nx; rl++; }
        }
      }
      float *gy = a.y + (rowb + k0) * p;
      int rl = lane / p, o = lane % p;
      const int drl = 64 / p, dop = 64 % p;
      for (int e = lane; e < rows * p; e += 64) {
        gy[e] = sy[rl * p + o + rl / V];
        rl += drl;
        o += dop;
        if (o >= p) { o -= p; rl++; }
      }
      ls_sync();  // the next round rewrites the stage
    }
    // state after the round's last step (only a sequence's final round can
    // end inside a lane; nothing reads the state after it)
    const int last = (k_end - 1 - k0) / V;
#pragma unroll
    for (int r = 0; r < NX; r++) st[r] = __shfl(z[r], last, 64);
  }
  if constexpr (!APPLY) {
    if (lane < nx) {
      float v = 0.f;
#pragma unroll
      for (int r = 0; r < NX; r++) v = lane == r ? st[r] : v;
      a.agg[(size_t)chunk * LS_W + lane] = v;
    }
  }
}

// One wavefront per sequence; lanes take 64 chunks at a time.
template <int NX>
__global__ __launch_bounds__(64) void k_lsim_carry(const LsimArgs a) {
  const int lane = threadIdx.x, b = blockIdx.x;
  const int nx = a.nx, cps = a.cps;
  // multipliers (Pc)^(2^i), Pc = Ad^(64 V LS_R) = P^LS_R: slots 8 + LS_LOGR + i
  __shared__ float P[6 * LS_MAT];
  for (int e = lane; e < 6 * LS_MAT; e += 64) P[e] = a.table[(8 + LS_LOGR) * LS_MAT + e];
  ls_sync();
  float c[NX];  // state entering the current group of chunks
#pragma unroll
  for (int r = 0; r < NX; r++) c[r] = (a.x0 && r < nx) ? a.x0[(size_t)b * nx + r] : 0.f;
  // aggregates of the group at g0 (clamped addresses; lanes past cps are zeroed)
  auto load = [&](int g0, float (&e)[NX]) __attribute__((always_inline)) {
    const size_t ch = (size_t)b * cps + min(g0 + lane, cps - 1);
#pragma unroll
    for (int r = 0; r < NX; r++) e[r] = a.agg[ch * LS_W + min(r, nx - 1)];
#pragma unroll
    for (int r = 0; r < NX; r++) e[r] = (g0 + lane < cps && r < nx) ? e[r] : 0.f;
  };
  float en[NX];
  load(0, en);
  for (int g0 = 0; g0 < cps; g0 += 64) {
    const int jj = g0 + lane;
    float e[NX];
#pragma unroll
    for (int r = 0; r < NX; r++) e[r] = en[r];
    load(g0 + 64 < cps ? g0 + 64 : g0, en);
    float pc[NX];
    ls_mv<NX>(P, c, pc);
    if (lane == 0) {
#pragma unroll
      for (int r = 0; r < NX; r++) e[r] += pc[r];
    }
    ls_wave_scan<NX>(P, e);  // e = state after chunk jj
#pragma unroll
    for (int r = 0; r < NX; r++) {
      const float prev = __shfl_up(e[r], 1, 64);  // state entering chunk jj
      if (jj < cps && r < nx) a.carry[((size_t)b * cps + jj) * LS_W + r] = lane == 0 ? c[r] : prev;
    }
#pragma unroll
    for (int r = 0; r < NX; r++) c[r] = __shfl(e[r], 63, 64);
  }
}

template <int NX, int MP>
static hipError_t lsim_run(const LsimArgs &a, hipStream_t s) {
  hipLaunchKernelGGL((k_lsim_pass<NX, MP, false>), dim3(a.nchunks), dim3(64), 0, s, a);
  hipLaunchKernelGGL(k_lsim_carry<NX>, dim3(a.B), dim3(64), 0, s, a);
  hipLaunchKernelGGL((k_lsim_pass<NX, MP, true>), dim3(a.nchunks), dim3(64), ls_stage_bytes(NX, ls_v(MP), a.p), s,
                     a);
  return hipGetLastError();
}

template <int NX>
static hipError_t lsim_run_m(const LsimArgs &a, hipStream_t s) {
  if (a.m <= 1) return lsim_run<NX, 1>(a, s);
  if (a.m <= 2) return lsim_run<NX, 2>(a, s);
  if (a.m <= 4) return lsim_run<NX, 4>(a, s);
  return lsim_run<NX, 8>(a, s);
}

hipError_t launch_lsim(LsimArgs &a, hipStream_t s) {
  a.V = ls_v(ls_mpad(a.m));
  const int L = lsim_chunk_len(a.m);
  a.cps = (a.T + L - 1) / L;
  a.nchunks = a.cps * a.B;
  if (a.nx + a.m <= 8) hipLaunchKernelGGL(k_lsim_disc<8>, dim3(1), dim3(64), 0, s, a);
  else hipLaunchKernelGGL(k_lsim_disc<16>, dim3(1), dim3(64), 0, s, a);
  if (a.nx <= 1) return lsim_run_m<1>(a, s);
  if (a.nx <= 2) return lsim_run_m<2>(a, s);
  if (a.nx <= 4) return lsim_run_m<4>(a, s);
  return lsim_run_m<8>(a, s);
}

}  // namespace pr

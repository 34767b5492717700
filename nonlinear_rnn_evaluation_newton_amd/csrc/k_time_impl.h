// Time-parallel kernels for small dense states (n <= 8, padded to N):
// one fused Newton sweep per launch (cell + Jacobian + residual + affine scan
// + update + convergence measure), the fused adjoint pass, and the standalone
// affine scan.
//
// A sweep evaluates f_t and J_t = df/dh at every step in parallel, forms
// r_t = f_t - h_t and solves dh_t = J_t dh_{t-1} + r_t with an associative
// scan of the operator (J_t, r_t) ("Parallelizing non-linear sequential models
// over the sequence length", Approach; Para-Seq README, Background).
//
// Layout: lanes run along time.  A tile is 4 wavefronts x Q groups x 64 lanes
// x V consecutive steps; a lane composes its V steps serially, the wavefront
// scans the 64 lane operators in DPP registers, the 4 wavefronts combine
// through LDS, and tiles of a sequence chain through a decoupled look-back.
//
// Scheduling: a persistent grid (every block resident at once) walks the
// tiles round-robin in increasing order, so a tile only ever waits on tiles
// that resident blocks have already reached; no tile counter is needed (a
// device-wide atomic counter serialises block starts on this part).  Each
// block prefetches its next tile's inputs before it waits in the look-back.
//
// The iterate h is updated in place; the one value a tile needs from its
// predecessor (h at its first step - 1) is kept from the previous sweep in a
// small boundary buffer.
#pragma once

#include <algorithm>

#include "cells_dense.h"
#include "internal.h"

namespace pr {

template <int N>
struct TimeGeom;
template <>
struct TimeGeom<1> {
  static constexpr int V = 4, Q = 4;
};
template <>
struct TimeGeom<2> {
  static constexpr int V = 2, Q = 4;
};
template <>
struct TimeGeom<4> {
  static constexpr int V = 1, Q = 2;
};
template <>
struct TimeGeom<8> {
  static constexpr int V = 1, Q = 1;
};

template <int N>
constexpr int time_tile_c() {
  return 4 * TimeGeom<N>::Q * 64 * TimeGeom<N>::V;
}

// Load steps t_lo .. t_lo+V-1 of a row of `width`-float records (padded to W).
// Steps outside [0, T) read as zeros.  The vector path needs V*W == 4,
// width == W, 16-byte alignment and T % V == 0 (checked by the caller).
template <int V, int W>
__device__ inline void load_steps(const float *__restrict__ row, int t_lo, int T, int width, bool vec,
                                  float (&out)[V][W]) {
  float *o = &out[0][0];
  if constexpr (V * W == 4) {
    if (vec) {
      if (t_lo >= 0 && t_lo < T) {
        float4 v4 = *reinterpret_cast<const float4 *>(row + (size_t)t_lo * W);
        o[0] = v4.x; o[1] = v4.y; o[2] = v4.z; o[3] = v4.w;
      } else {
        o[0] = o[1] = o[2] = o[3] = 0.f;
      }
      return;
    }
  }
#pragma unroll
  for (int v = 0; v < V; v++) {
    const int t = t_lo + v;
#pragma unroll
    for (int i = 0; i < W; i++) out[v][i] = (i < width && t >= 0 && t < T) ? row[(size_t)t * width + i] : 0.f;
  }
}

template <int V, int W>
__device__ inline void store_steps(float *__restrict__ row, int t_lo, int T, int width, bool vec,
                                   const float (&in)[V][W]) {
  const float *o = &in[0][0];
  if constexpr (V * W == 4) {
    if (vec) {
      if (t_lo >= 0 && t_lo < T) *reinterpret_cast<float4 *>(row + (size_t)t_lo * W) = make_float4(o[0], o[1], o[2], o[3]);
      return;
    }
  }
#pragma unroll
  for (int v = 0; v < V; v++) {
    const int t = t_lo + v;
    if (t >= 0 && t < T) {
#pragma unroll
      for (int i = 0; i < W; i++)
        if (i < width) row[(size_t)t * width + i] = in[v][i];
    }
  }
}

// Scan of the lane operators ops[q] (group q of this lane) over the tile.
// ex[q] receives the composition of every operator of the tile before group
// q; tot the tile aggregate.  Contains one __syncthreads.
template <int N, int Q>
__device__ inline void tile_scan(const Op<N> (&ops)[Q], Op<N> (&ex)[Q], Op<N> &tot, Op<N> *s_wtot) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  Op<N> run = op_identity<N>();
#pragma unroll
  for (int q = 0; q < Q; q++) {
    Op<N> inc = wave_scan_incl<N>(ops[q]);
    ex[q] = compose(wave_shift1<N>(inc), run);
    run = compose(wave_last<N>(inc), run);
  }
  if (lane == 0) s_wtot[wid] = run;
  __syncthreads();
  Op<N> pre = op_identity<N>();
  for (int w = 0; w < wid; w++) pre = compose(s_wtot[w], pre);
#pragma unroll
  for (int q = 0; q < Q; q++) ex[q] = compose(ex[q], pre);
  tot = compose(s_wtot[3], compose(s_wtot[2], compose(s_wtot[1], s_wtot[0])));
}

// Decoupled look-back for tile j of one sequence (descriptor base pointers
// already offset to that sequence), run by all 64 lanes of wavefront 0.
// Publishes the tile aggregate, reads up to 64 predecessors per round trip
// (lane l holds tile wend - 63 + l, so lane 63 is the nearest; a lane issues
// its inclusive and aggregate loads together), composes the aggregates after
// the nearest inclusive prefix in the window, and publishes this tile's
// inclusive prefix.  carry receives the state after tile j - 1.
template <int N>
__device__ inline void lookback(const Op<N> &tot, int j, int k, unsigned long long *agg, unsigned long long *incl,
                                float *carry, SolveState *st) {
  constexpr int AW = N * N + N;
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < N; i++) carry[i] = 0.f;
  if (j > 0) {
    if (lane == 0) {
#pragma unroll
      for (int i = 0; i < N * N; i++) desc_put(agg + (size_t)j * AW + i, tag_agg(k), tot.A[i]);
#pragma unroll
      for (int i = 0; i < N; i++) desc_put(agg + (size_t)j * AW + N * N + i, tag_agg(k), tot.b[i]);
    }
    Op<N> acc = op_identity<N>();
    int wend = j - 1, spins = 0;
    while (true) {
      const int p = wend - 63 + lane;
      unsigned long long wi[N], wa[AW];
      if (p >= 0) {
#pragma unroll
        for (int i = 0; i < N; i++) wi[i] = ld_agent64(incl + (size_t)p * N + i);
#pragma unroll
        for (int i = 0; i < AW; i++) wa[i] = ld_agent64(agg + (size_t)p * AW + i);
      } else {
#pragma unroll
        for (int i = 0; i < N; i++) wi[i] = 0;
#pragma unroll
        for (int i = 0; i < AW; i++) wa[i] = 0;
      }
      bool hi = p >= 0, ha = p >= 0;
#pragma unroll
      for (int i = 0; i < N; i++) hi = hi && (unsigned)(wi[i] >> 32) == tag_incl(k);
#pragma unroll
      for (int i = 0; i < AW; i++) ha = ha && (unsigned)(wa[i] >> 32) == tag_agg(k);
      const unsigned long long bi = __ballot(hi);
      const int m = bi ? 63 - __clzll((long long)bi) : -1;  // nearest tile with an inclusive prefix
      const bool ok = !(lane > m && p >= 0) || ha;
      if (!__all(ok)) {
        if (++spins > PR_SPIN_LIMIT) {  // reported by the host; a NaN carry poisons the rest
          if (lane == 0) spin_fault(st);
          acc = op_identity<N>();
#pragma unroll
          for (int i = 0; i < N; i++) acc.b[i] = __builtin_nanf("");
          break;
        }
        __builtin_amdgcn_s_sleep(1);
        continue;
      }
      Op<N> o = op_identity<N>();
      if (lane == m) {
#pragma unroll
        for (int i = 0; i < N * N; i++) o.A[i] = 0.f;
#pragma unroll
        for (int i = 0; i < N; i++) o.b[i] = __uint_as_float((unsigned)wi[i]);
      } else if (lane > m && p >= 0) {
#pragma unroll
        for (int i = 0; i < N * N; i++) o.A[i] = __uint_as_float((unsigned)wa[i]);
#pragma unroll
        for (int i = 0; i < N; i++) o.b[i] = __uint_as_float((unsigned)wa[N * N + i]);
      }
      acc = compose(acc, wave_last<N>(wave_scan_incl<N>(o)));
      if (m >= 0) break;
      wend -= 64;
    }
#pragma unroll
    for (int i = 0; i < N; i++) carry[i] = acc.b[i];  // acc ends in a constant operator: acc(.) = acc.b
  }
  if (lane == 0) {
    float inc[N];
    op_apply(tot, carry, inc);
#pragma unroll
    for (int i = 0; i < N; i++) desc_put(incl + (size_t)j * N + i, tag_incl(k), inc[i]);
  }
}

// Stop rule on the previous sweep's measure (run by wavefront 0 at the start
// of sweep k >= 2).  Block 0 also finalises delta_{k-1} into the history and
// clears the shards sweep k + 1 will use.  Returns true when the solve has
// stopped (every block then exits).
__device__ inline bool sweep_stopped(const TimeArgs &a, int *s_stop) {
  const int k = a.k;
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int stop = ld_agent(&a.st->stopped) != 0;
    if (!stop && k >= 2) {
      unsigned d = ld_agent(&a.st->dslot[(k - 1) & 3][lane]);
      d = wave_max_u32(d);
      int status;
      if (stop_rule(__uint_as_float(d), k - 1, a.tol, a.T, a.max_iters, &status)) {
        stop = 1;
        if (blockIdx.x == 0 && lane == 0) {
          st_agent((unsigned *)&a.st->iters, (unsigned)(k - 1));
          st_agent((unsigned *)&a.st->status, (unsigned)status);
          st_agent(&a.st->stopped, 1u);
        }
      }
      if (blockIdx.x == 0 && lane == 0) st_agent(&a.st->hist[(k - 1) % PR_HIST], d);
    }
    if (!stop && blockIdx.x == 0) st_agent(&a.st->dslot[(k + 1) & 3][lane], 0u);
    if (lane == 0) *s_stop = stop;
  }
  __syncthreads();
  return *s_stop != 0;
}

template <int N, int G, int DX>
__device__ inline void stage_dense_weights(const TimeArgs &a, float *sWh, float *sbh, float *sWx, float *sbx) {
  const int n = a.n, d = a.d;
  for (int e = threadIdx.x; e < G * N * N; e += blockDim.x) {
    const int g = e / (N * N), r = (e / N) % N, c = e % N;
    sWh[e] = (r < n && c < n) ? a.Wh[((size_t)g * n + r) * n + c] : 0.f;
  }
  for (int e = threadIdx.x; e < G * N * DX; e += blockDim.x) {
    const int g = e / (N * DX), r = (e / DX) % N, c = e % DX;
    sWx[e] = (r < n && c < d) ? a.Wx[((size_t)g * n + r) * d + c] : 0.f;
  }
  for (int e = threadIdx.x; e < G * N; e += blockDim.x) {
    const int g = e / N, r = e % N;
    sbh[e] = (r < n && a.bh) ? a.bh[(size_t)g * n + r] : 0.f;
    sbx[e] = (r < n && a.bx) ? a.bx[(size_t)g * n + r] : 0.f;
  }
}

template <int N, int G, int DX>
__device__ inline void input_proj(const float *sWx, const float *sbx, const float *xt, float *U) {
#pragma unroll
  for (int j = 0; j < G * N; j++) {
    float u = sbx[j];
#pragma unroll
    for (int c = 0; c < DX; c++) u = fmaf(sWx[j * DX + c], xt[c], u);
    U[j] = u;
  }
}

// ---------------------------------------------------------------------------
// one Newton sweep
// ---------------------------------------------------------------------------
template <int N, int DX, int V, int Q>
struct SweepRaw {
  float h[Q][V][N];   // current iterate
  float x[Q][V][DX];  // inputs
  float sp[Q][N];     // state before each group's first step
};

// Issue the loads of tile `id` (no waits until the values are used).
template <int N, int DX, int V, int Q>
__device__ inline void sweep_load(const TimeArgs &a, int id, bool vec_h, bool vec_x, SweepRaw<N, DX, V, Q> &R) {
  constexpr int TILE = 4 * Q * 64 * V;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, k = a.k;
  const int B = a.B, T = a.T, n = a.n, d = a.d;
  const int j = id / B, b = id % B, L = b * a.tiles_per_seq + j;
  const int t0 = j * TILE;
  const float *hrow = a.h + (size_t)b * T * n;
  const float *xrow = a.x + (size_t)b * T * d;
#pragma unroll
  for (int q = 0; q < Q; q++) {
    const int base = t0 + ((wid * Q + q) * 64 + lane) * V;
    if (k >= 2) {
      load_steps<V, N>(hrow, base, T, n, vec_h, R.h[q]);
    } else {
#pragma unroll
      for (int v = 0; v < V; v++)
#pragma unroll
        for (int i = 0; i < N; i++) R.h[q][v][i] = 0.f;
    }
    load_steps<V, DX>(xrow, base, T, d, vec_x, R.x[q]);
#pragma unroll
    for (int i = 0; i < N; i++) {
      float s = 0.f;
      if (i < n && base < T) {
        if (base == 0) s = a.h0 ? a.h0[(size_t)b * n + i] : 0.f;
        else if (k == 1) s = 0.f;
        else if (base == t0) s = a.bnd[((size_t)((k - 1) & 1) * a.ntiles + (L - 1)) * N + i];
        else s = hrow[(size_t)(base - 1) * n + i];
      }
      R.sp[q][i] = s;
    }
  }
}

template <int N, int CELL, int DX>
__global__ __launch_bounds__(256) void k_time_sweep(const TimeArgs a) {
  constexpr int V = TimeGeom<N>::V, Q = TimeGeom<N>::Q, G = cell_gates(CELL), TILE = time_tile_c<N>();
  __shared__ float sWh[G * N * N], sbh[G * N], sWx[G * N * DX], sbx[G * N];
  __shared__ Op<N> s_wtot[4];
  __shared__ float s_carry[N];
  __shared__ int s_stop;
  __shared__ unsigned s_dmax[4];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, k = a.k;
  const int B = a.B, T = a.T, n = a.n, d = a.d;
  const bool vec_h = (a.vec_ok & 1) && n == N && (T % V) == 0;
  const bool vec_x = (a.vec_ok & 2) && d == DX && (T % V) == 0;

  SweepRaw<N, DX, V, Q> R;
  int id = blockIdx.x;
  if (id < a.ntiles) sweep_load(a, id, vec_h, vec_x, R);  // overlaps the stop check
  if (sweep_stopped(a, &s_stop)) return;
  stage_dense_weights<N, G, DX>(a, sWh, sbh, sWx, sbx);
  __syncthreads();

  unsigned dmax = 0;
  for (; id < a.ntiles; id += gridDim.x) {
    const int j = id / B, b = id % B, L = b * a.tiles_per_seq + j;
    const int t0 = j * TILE;
    float *hrow = a.h + (size_t)b * T * n;

    float Jv[Q][V][N * N], rv[Q][V][N], hv[Q][V][N];
    Op<N> ops[Q];
#pragma unroll
    for (int q = 0; q < Q; q++) {
      const int base = t0 + ((wid * Q + q) * 64 + lane) * V;
      float sp[N];
#pragma unroll
      for (int i = 0; i < N; i++) sp[i] = R.sp[q][i];
      ops[q] = op_identity<N>();
#pragma unroll
      for (int v = 0; v < V; v++) {
#pragma unroll
        for (int i = 0; i < N; i++) hv[q][v][i] = R.h[q][v][i];
        if (base + v < T) {
          float U[G * N], f[N];
          input_proj<N, G, DX>(sWx, sbx, R.x[q][v], U);
          dense_cell<N, CELL>(sp, U, sWh, sbh, f, Jv[q][v]);
          if (a.approx != APX_NEWTON) {  // quasi-DEER keeps the diagonal, Jacobi nothing
#pragma unroll
            for (int i = 0; i < N; i++)
#pragma unroll
              for (int m = 0; m < N; m++)
                if (a.approx == APX_ZERO || m != i) Jv[q][v][i * N + m] = 0.f;
          }
          Op<N> e;
#pragma unroll
          for (int i = 0; i < N; i++) {
            rv[q][v][i] = f[i] - hv[q][v][i];
            e.b[i] = rv[q][v][i];
            sp[i] = hv[q][v][i];
          }
#pragma unroll
          for (int i = 0; i < N * N; i++) e.A[i] = Jv[q][v][i];
          ops[q] = compose(e, ops[q]);
        }
      }
    }

    Op<N> ex[Q], tot;
    tile_scan<N, Q>(ops, ex, tot, s_wtot);
    const int nid = id + gridDim.x;
    if (nid < a.ntiles) sweep_load(a, nid, vec_h, vec_x, R);  // prefetch while waiting
    if (wid == 0) {
      float c[N];
      lookback<N>(tot, j, k, a.agg + (size_t)b * a.tiles_per_seq * (N * N + N),
                  a.incl + (size_t)b * a.tiles_per_seq * N, c, a.st);
      if (lane == 0) {
#pragma unroll
        for (int i = 0; i < N; i++) s_carry[i] = c[i];
      }
    }
    __syncthreads();

#pragma unroll
    for (int q = 0; q < Q; q++) {
      const int base = t0 + ((wid * Q + q) * 64 + lane) * V;
      float dh[N], carry[N], hn[V][N];
#pragma unroll
      for (int i = 0; i < N; i++) carry[i] = s_carry[i];
      op_apply(ex[q], carry, dh);
#pragma unroll
      for (int v = 0; v < V; v++) {
        float nd[N];
#pragma unroll
        for (int i = 0; i < N; i++) {
          float acc = rv[q][v][i];
#pragma unroll
          for (int m = 0; m < N; m++) acc = fmaf(Jv[q][v][i * N + m], dh[m], acc);
          nd[i] = acc;
        }
        const bool valid = base + v < T;
#pragma unroll
        for (int i = 0; i < N; i++) {
          dh[i] = nd[i];
          hn[v][i] = hv[q][v][i] + nd[i];
          if (valid && i < n) {
            unsigned u = __float_as_uint(fabsf(nd[i]));
            dmax = u > dmax ? u : dmax;
          }
        }
      }
      store_steps<V, N>(hrow, base, T, n, vec_h, hn);
      if (wid == 3 && q == Q - 1 && lane == 63 && base + V - 1 < T) {
#pragma unroll
        for (int i = 0; i < N; i++) a.bnd[((size_t)(k & 1) * a.ntiles + L) * N + i] = hn[V - 1][i];
      }
    }
  }
  dmax = wave_max_u32(dmax);
  if (lane == 0) s_dmax[wid] = dmax;
  __syncthreads();
  if (tid == 0) {
    unsigned m = s_dmax[0];
    for (int w = 1; w < 4; w++) m = s_dmax[w] > m ? s_dmax[w] : m;
    max_agent(&a.st->dslot[k & 3][blockIdx.x % PR_DSHARDS], m);
  }
}

// ---------------------------------------------------------------------------
// adjoint: lam_t = g_t + J_{t+1}^T lam_{t+1} by a reverse-time scan, then the
// chain rule through each cell for dx, dh0 and per-block weight partials
// ---------------------------------------------------------------------------
template <int N, int G, int DX>
__host__ __device__ constexpr int time_part_c() {
  return G * N * DX + G * N + G * N * N + G * N;
}

template <int N, int DX, int V, int Q>
struct AdjRaw {
  float h[Q][V][N], g[Q][V][N], x[Q][V][DX];
  float xn[Q][DX];  // x at the step after each group
  float hp[Q][N];   // h at the step before each group
};

// Scan order runs backwards in time: scan position s <-> t = T - 1 - s.
// Group (w, q, lane) of tile j covers times [tlo, tlo + V).
template <int N, int DX, int V, int Q>
__device__ inline void adj_load(const TimeArgs &a, int id, bool vec_h, bool vec_x, bool vec_g,
                                AdjRaw<N, DX, V, Q> &R) {
  constexpr int TILE = 4 * Q * 64 * V;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int B = a.B, T = a.T, n = a.n, d = a.d;
  const int j = id / B, b = id % B;
  const float *hrow = a.h + (size_t)b * T * n;
  const float *grow = a.g + (size_t)b * T * n;
  const float *xrow = a.x + (size_t)b * T * d;
#pragma unroll
  for (int q = 0; q < Q; q++) {
    const int s0 = j * TILE + ((wid * Q + q) * 64 + lane) * V;
    const int tlo = T - s0 - V;
    load_steps<V, N>(hrow, tlo, T, n, vec_h, R.h[q]);
    load_steps<V, N>(grow, tlo, T, n, vec_g, R.g[q]);
    load_steps<V, DX>(xrow, tlo, T, d, vec_x, R.x[q]);
#pragma unroll
    for (int c = 0; c < DX; c++)
      R.xn[q][c] = (c < d && tlo + V < T && tlo + V >= 0) ? xrow[(size_t)(tlo + V) * d + c] : 0.f;
#pragma unroll
    for (int i = 0; i < N; i++) R.hp[q][i] = (i < n && tlo >= 1 && tlo <= T) ? hrow[(size_t)(tlo - 1) * n + i] : 0.f;
  }
}

template <int N, int CELL, int DX>
__global__ __launch_bounds__(256) void k_time_adjoint(const TimeArgs a) {
  constexpr int V = TimeGeom<N>::V, Q = TimeGeom<N>::Q, G = cell_gates(CELL), TILE = time_tile_c<N>();
  constexpr int P = time_part_c<N, G, DX>();
  __shared__ float sWh[G * N * N], sbh[G * N], sWx[G * N * DX], sbx[G * N];
  __shared__ Op<N> s_wtot[4];
  __shared__ float s_carry[N];
  __shared__ float s_red[4][P];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int B = a.B, T = a.T, n = a.n, d = a.d;
  const bool vec_h = (a.vec_ok & 1) && n == N && (T % V) == 0;
  const bool vec_x = (a.vec_ok & 2) && d == DX && (T % V) == 0;
  const bool vec_g = (a.vec_ok & 4) && n == N && (T % V) == 0;
  const bool vec_l = (a.vec_ok & 8) && n == N && (T % V) == 0;

  AdjRaw<N, DX, V, Q> R;
  int id = blockIdx.x;
  if (id < a.ntiles) adj_load(a, id, vec_h, vec_x, vec_g, R);
  stage_dense_weights<N, G, DX>(a, sWh, sbh, sWx, sbx);
  __syncthreads();
  float hz[N];  // h0 of the current sequence
  float acc[P];
#pragma unroll
  for (int p = 0; p < P; p++) acc[p] = 0.f;
  float *aWx = acc, *abx = acc + G * N * DX, *aWh = abx + G * N, *abh = aWh + G * N * N;

  for (; id < a.ntiles; id += gridDim.x) {
    const int j = id / B, b = id % B;
#pragma unroll
    for (int i = 0; i < N; i++) hz[i] = (i < n && a.h0) ? a.h0[(size_t)b * n + i] : 0.f;
    float Av[Q][V][N * N], gv[Q][V][N], hv[Q][V][N], xv[Q][V][DX], hp[Q][N];
    Op<N> ops[Q];
#pragma unroll
    for (int q = 0; q < Q; q++) {
      const int s0 = j * TILE + ((wid * Q + q) * 64 + lane) * V;
      const int tlo = T - s0 - V;
#pragma unroll
      for (int i = 0; i < N; i++) hp[q][i] = R.hp[q][i];
#pragma unroll
      for (int v = 0; v < V; v++) {
#pragma unroll
        for (int i = 0; i < N; i++) { hv[q][v][i] = R.h[q][v][i]; gv[q][v][i] = R.g[q][v][i]; }
#pragma unroll
        for (int c = 0; c < DX; c++) xv[q][v][c] = R.x[q][v][c];
      }
      ops[q] = op_identity<N>();
#pragma unroll
      for (int v = 0; v < V; v++) {
        const int e = V - 1 - v;  // storage index of time t
        const int t = tlo + e;
        if (t >= 0 && t < T) {
          float J[N * N];
          if (t + 1 < T) {
            float U[G * N], f[N];
            input_proj<N, G, DX>(sWx, sbx, e + 1 < V ? xv[q][e + 1] : R.xn[q], U);
            dense_cell<N, CELL>(hv[q][e], U, sWh, sbh, f, J);
          } else {
#pragma unroll
            for (int i = 0; i < N * N; i++) J[i] = 0.f;
          }
          Op<N> o;
#pragma unroll
          for (int r = 0; r < N; r++) {
#pragma unroll
            for (int c = 0; c < N; c++) o.A[r * N + c] = J[c * N + r];  // transpose
            o.b[r] = gv[q][e][r];
          }
#pragma unroll
          for (int i = 0; i < N * N; i++) Av[q][e][i] = o.A[i];
          ops[q] = compose(o, ops[q]);
        }
      }
    }

    Op<N> ex[Q], tot;
    tile_scan<N, Q>(ops, ex, tot, s_wtot);
    const int nid = id + gridDim.x;
    if (nid < a.ntiles) adj_load(a, nid, vec_h, vec_x, vec_g, R);  // prefetch while waiting
    if (wid == 0) {
      float c[N];
      lookback<N>(tot, j, 1, a.agg + (size_t)b * a.tiles_per_seq * (N * N + N),
                  a.incl + (size_t)b * a.tiles_per_seq * N, c, a.st);
      if (lane == 0) {
#pragma unroll
        for (int i = 0; i < N; i++) s_carry[i] = c[i];
      }
    }
    __syncthreads();

#pragma unroll
    for (int q = 0; q < Q; q++) {
      const int s0 = j * TILE + ((wid * Q + q) * 64 + lane) * V;
      const int tlo = T - s0 - V;
      float lam[N], carry[N];
#pragma unroll
      for (int i = 0; i < N; i++) carry[i] = s_carry[i];
      op_apply(ex[q], carry, lam);
      float lv[V][N];
#pragma unroll
      for (int v = 0; v < V; v++) {
        const int e = V - 1 - v;
        const int t = tlo + e;
        float nl[N];
#pragma unroll
        for (int i = 0; i < N; i++) {
          float x = gv[q][e][i];
#pragma unroll
          for (int m = 0; m < N; m++) x = fmaf(Av[q][e][i * N + m], lam[m], x);
          nl[i] = x;
        }
#pragma unroll
        for (int i = 0; i < N; i++) { lam[i] = nl[i]; lv[e][i] = nl[i]; }
        if (t >= 0 && t < T) {
          const float *sp = t == 0 ? hz : (e > 0 ? hv[q][e - 1] : hp[q]);
          float U[G * N], ds[N], dU[G * N];
          input_proj<N, G, DX>(sWx, sbx, xv[q][e], U);
          dense_cell_vjp<N, CELL>(sp, U, lam, sWh, sbh, ds, dU, aWh, abh);
#pragma unroll
          for (int jg = 0; jg < G * N; jg++) {
            abx[jg] += dU[jg];
#pragma unroll
            for (int c = 0; c < DX; c++) aWx[jg * DX + c] = fmaf(dU[jg], xv[q][e][c], aWx[jg * DX + c]);
          }
          if (a.dx) {
#pragma unroll
            for (int c = 0; c < DX; c++) {
              if (c < d) {
                float s = 0.f;
#pragma unroll
                for (int jg = 0; jg < G * N; jg++) s = fmaf(sWx[jg * DX + c], dU[jg], s);
                a.dx[((size_t)b * T + t) * d + c] = s;
              }
            }
          }
          if (t == 0 && a.dh0) {
#pragma unroll
            for (int i = 0; i < N; i++)
              if (i < n) a.dh0[(size_t)b * n + i] = ds[i];
          }
        }
      }
      if (a.lam) store_steps<V, N>(a.lam + (size_t)b * T * n, tlo, T, n, vec_l, lv);
    }
  }
  // block reduction of the weight-gradient partials
#pragma unroll
  for (int p = 0; p < P; p++) {
    float v = wave_total(acc[p]);
    if (lane == 0) s_red[wid][p] = v;
  }
  __syncthreads();
  for (int p = tid; p < P; p += 256)
    a.part[(size_t)blockIdx.x * P + p] = (s_red[0][p] + s_red[1][p]) + (s_red[2][p] + s_red[3][p]);
}

// Sum the per-block partials in fp64, in block order, and scatter to the
// unpadded fp32 outputs.
template <int N, int G, int DX>
__global__ __launch_bounds__(256) void k_time_reduce(const float *part, int nparts, int n, int d, float *dWx,
                                                     float *dbx, float *dWh, float *dbh) {
  constexpr int P = time_part_c<N, G, DX>();
  __shared__ double s[256];
  const int p = blockIdx.x;
  double acc = 0.0;
  for (int L = threadIdx.x; L < nparts; L += 256) acc += (double)part[(size_t)L * P + p];
  s[threadIdx.x] = acc;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) s[threadIdx.x] += s[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x != 0) return;
  const float v = (float)s[0];
  int q = p;
  if (q < G * N * DX) {
    const int jg = q / DX, c = q % DX, g = jg / N, i = jg % N;
    if (dWx && i < n && c < d) dWx[((size_t)g * n + i) * d + c] = v;
    return;
  }
  q -= G * N * DX;
  if (q < G * N) {
    const int g = q / N, i = q % N;
    if (dbx && i < n) dbx[(size_t)g * n + i] = v;
    return;
  }
  q -= G * N;
  if (q < G * N * N) {
    const int g = q / (N * N), i = (q / N) % N, c = q % N;
    if (dWh && i < n && c < n) dWh[((size_t)g * n + i) * n + c] = v;
    return;
  }
  q -= G * N * N;
  {
    const int g = q / N, i = q % N;
    if (dbh && i < n) dbh[(size_t)g * n + i] = v;
  }
}

// ---------------------------------------------------------------------------
// standalone affine scan: y_t = A_t y_{t-1} + b_t (or reverse time)
// ---------------------------------------------------------------------------
template <int N>
__global__ __launch_bounds__(256) void k_time_scan(const ScanArgs a) {
  constexpr int V = TimeGeom<N>::V, Q = TimeGeom<N>::Q, TILE = time_tile_c<N>();
  __shared__ Op<N> s_wtot[4];
  __shared__ float s_carry[N];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int B = a.B, T = a.T, n = a.n;
  for (int id = blockIdx.x; id < a.ntiles; id += gridDim.x) {
    const int j = id / B, b = id % B;
    Op<N> ops[Q], el[Q][V];
#pragma unroll
    for (int q = 0; q < Q; q++) {
      const int s0 = j * TILE + ((wid * Q + q) * 64 + lane) * V;
      ops[q] = op_identity<N>();
#pragma unroll
      for (int v = 0; v < V; v++) {
        const int sidx = s0 + v;
        const int t = a.reverse ? T - 1 - sidx : sidx;
        Op<N> o = op_identity<N>();
        if (sidx < T) {
          const size_t e = (size_t)b * T + t;
#pragma unroll
          for (int r = 0; r < N; r++) {
#pragma unroll
            for (int c = 0; c < N; c++) o.A[r * N + c] = (r < n && c < n) ? a.A[(e * n + r) * n + c] : 0.f;
            o.b[r] = r < n ? a.b[e * n + r] : 0.f;
          }
          ops[q] = compose(o, ops[q]);
        }
        el[q][v] = o;
      }
    }
    Op<N> ex[Q], tot;
    tile_scan<N, Q>(ops, ex, tot, s_wtot);
    if (wid == 0) {
      float c[N];
      lookback<N>(tot, j, 1, a.agg + (size_t)b * a.tiles_per_seq * (N * N + N),
                  a.incl + (size_t)b * a.tiles_per_seq * N, c, a.st);
      if (lane == 0) {
#pragma unroll
        for (int i = 0; i < N; i++) s_carry[i] = c[i];
      }
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < Q; q++) {
      const int s0 = j * TILE + ((wid * Q + q) * 64 + lane) * V;
      float y[N], carry[N];
#pragma unroll
      for (int i = 0; i < N; i++) carry[i] = s_carry[i];
      op_apply(ex[q], carry, y);
#pragma unroll
      for (int v = 0; v < V; v++) {
        const int sidx = s0 + v;
        float ny[N];
        op_apply(el[q][v], y, ny);
#pragma unroll
        for (int i = 0; i < N; i++) y[i] = ny[i];
        if (sidx < T) {
          const int t = a.reverse ? T - 1 - sidx : sidx;
          const size_t e = (size_t)b * T + t;
#pragma unroll
          for (int i = 0; i < N; i++)
            if (i < n) a.y[e * n + i] = y[i];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Quasi-ELK producer for the small dense cells (Gonzalez et al. abstract:
// quasi-ELK keeps the Jacobian's diagonal): at the current iterate, the
// diagonal of J_t and the residual r_t = f_t - h_t of every step,
// [row][d (n) | r (n)] fp32, one thread per step.  Opens the sweep.
// ---------------------------------------------------------------------------
template <int N, int CELL, int DX>
__global__ __launch_bounds__(256) void k_time_elk_jr(const TimeArgs a, float *jr) {
  constexpr int G = cell_gates(CELL);
  __shared__ float sWh[G * N * N], sbh[G * N], sWx[G * N * DX], sbx[G * N];
  __shared__ int s_stop;
  if (sweep_open(a.st, a.k, a.tol, a.T, a.max_iters, &s_stop)) return;
  stage_dense_weights<N, G, DX>(a, sWh, sbh, sWx, sbx);
  __syncthreads();
  const int n = a.n, d = a.d, T = a.T;
  const size_t rows = (size_t)a.B * T;
  const bool first = a.k == 1;  // the iterate is h = 0 before sweep 1
  for (size_t row = (size_t)blockIdx.x * blockDim.x + threadIdx.x; row < rows; row += (size_t)gridDim.x * blockDim.x) {
    const int t = (int)(row % T), b = (int)(row / T);
    float xt[DX], sp[N], hc[N], U[G * N], f[N], J[N * N];
#pragma unroll
    for (int c = 0; c < DX; c++) xt[c] = c < d ? a.x[row * d + c] : 0.f;
#pragma unroll
    for (int i = 0; i < N; i++) {
      float v = 0.f;
      if (i < n) {
        if (t > 0) v = first ? 0.f : a.h[(row - 1) * n + i];
        else if (a.h0) v = a.h0[(size_t)b * n + i];
      }
      sp[i] = v;
      hc[i] = (i < n && !first) ? a.h[row * n + i] : 0.f;
    }
    input_proj<N, G, DX>(sWx, sbx, xt, U);
    dense_cell<N, CELL>(sp, U, sWh, sbh, f, J);
    float *o = jr + row * 2 * n;
#pragma unroll
    for (int i = 0; i < N; i++) {
      if (i < n) {
        o[i] = J[i * N + i];
        o[n + i] = f[i] - hc[i];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// launch helpers
// ---------------------------------------------------------------------------
static inline int dx_pad(int d) { return d <= 1 ? 1 : d <= 2 ? 2 : d <= 4 ? 4 : 8; }

#define PR_DISPATCH_DX(d, ...)                                   \
  switch (dx_pad(d)) {                                           \
    case 1: { constexpr int DX = 1; __VA_ARGS__; } break;        \
    case 2: { constexpr int DX = 2; __VA_ARGS__; } break;        \
    case 4: { constexpr int DX = 4; __VA_ARGS__; } break;        \
    default: { constexpr int DX = 8; __VA_ARGS__; } break;       \
  }

#define PR_DISPATCH_N(Nv, ...)                                   \
  switch (Nv) {                                                  \
    case 1: { constexpr int N = 1; __VA_ARGS__; } break;         \
    case 2: { constexpr int N = 2; __VA_ARGS__; } break;         \
    case 4: { constexpr int N = 4; __VA_ARGS__; } break;         \
    case 8: { constexpr int N = 8; __VA_ARGS__; } break;         \
    default: return hipErrorInvalidValue;                        \
  }

// Launchers for one cell, instantiated in one translation unit per cell.
template <int CELL>
hipError_t time_sweep_cell(int Nv, const TimeArgs &a, hipStream_t s) {
  PR_DISPATCH_N(Nv, PR_DISPATCH_DX(a.d, {
    const int grid = persistent_grid<k_time_sweep<N, CELL, DX>>(a.ntiles);
    if (grid <= 0) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((k_time_sweep<N, CELL, DX>), dim3(grid), dim3(256), 0, s, a);
  }));
  return hipGetLastError();
}

template <int CELL>
hipError_t time_adjoint_cell(int Nv, TimeArgs &a, hipStream_t s) {
  PR_DISPATCH_N(Nv, PR_DISPATCH_DX(a.d, {
    const int grid = persistent_grid<k_time_adjoint<N, CELL, DX>>(a.ntiles);
    if (grid <= 0) return hipErrorInvalidConfiguration;
    a.nparts = grid;
    hipLaunchKernelGGL((k_time_adjoint<N, CELL, DX>), dim3(grid), dim3(256), 0, s, a);
  }));
  return hipGetLastError();
}

template <int CELL>
hipError_t time_reduce_cell(int Nv, const TimeArgs &a, const float *part, float *dWx, float *dbx, float *dWh,
                            float *dbh, hipStream_t s) {
  PR_DISPATCH_N(Nv, PR_DISPATCH_DX(a.d, {
    constexpr int G = cell_gates(CELL);
    constexpr int P = time_part_c<N, G, DX>();
    hipLaunchKernelGGL((k_time_reduce<N, G, DX>), dim3(P), dim3(256), 0, s, part, a.nparts, a.n, a.d, dWx, dbx,
                       dWh, dbh);
  }));
  return hipGetLastError();
}

hipError_t time_sweep_tanh(int Nv, const TimeArgs &a, hipStream_t s);
hipError_t time_sweep_gru(int Nv, const TimeArgs &a, hipStream_t s);
hipError_t time_sweep_linear(int Nv, const TimeArgs &a, hipStream_t s);
hipError_t time_adjoint_tanh(int Nv, TimeArgs &a, hipStream_t s);
hipError_t time_adjoint_gru(int Nv, TimeArgs &a, hipStream_t s);
hipError_t time_adjoint_linear(int Nv, TimeArgs &a, hipStream_t s);
hipError_t time_reduce_tanh(int Nv, const TimeArgs &a, const float *, float *, float *, float *, float *, hipStream_t);
hipError_t time_reduce_gru(int Nv, const TimeArgs &a, const float *, float *, float *, float *, float *, hipStream_t);
hipError_t time_reduce_linear(int Nv, const TimeArgs &a, const float *, float *, float *, float *, float *, hipStream_t);
hipError_t time_elk_jr_tanh(int Nv, const TimeArgs &a, float *jr, hipStream_t s);
hipError_t time_elk_jr_gru(int Nv, const TimeArgs &a, float *jr, hipStream_t s);
hipError_t time_elk_jr_linear(int Nv, const TimeArgs &a, float *jr, hipStream_t s);

template <int CELL>
hipError_t time_elk_jr_cell(int Nv, const TimeArgs &a, float *jr, hipStream_t s) {
  const size_t rows = (size_t)a.B * a.T;
  const unsigned grid = (unsigned)std::min<size_t>((rows + 255) / 256, 65536);
  PR_DISPATCH_N(Nv, PR_DISPATCH_DX(a.d, {
    hipLaunchKernelGGL((k_time_elk_jr<N, CELL, DX>), dim3(grid), dim3(256), 0, s, a, jr);
  }));
  return hipGetLastError();
}

}  // namespace pr

// Quasi-ELK sweeps: the Levenberg-Marquardt-damped quasi-Newton step solved
// as a Kalman smoother (Gonzalez et al. abstract: ELK stabilises DEER through
// the connection between Levenberg-Marquardt and Kalman smoothing; Para-Seq
// README, Main features: ELK and quasi-ELK solvers).
//
// With the Jacobian's diagonal d_t, every state entry i is a scalar model
//   dh_t = d_t dh_{t-1} + r_t + w_t,  w_t ~ N(0, 1),   0 = dh_t + v_t,
//   v_t ~ N(0, 1 / lambda),   dh_{-1} = 0,
// whose posterior mean is the damped step argmin ||L dh - r||^2 + lambda ||dh||^2.
// A sweep, after a producer has stored d_t and r_t at the current iterate
// ([row][d (S) | r (S)], fp32), runs three parallel scans over time, each in
// chunks of ELK_L steps (one wavefront per (sequence, chunk, 64 entries), lane
// = state entry), with a per-(sequence, entry) scan over the chunk aggregates:
//  1. the filter variance: P_t = (1 - K_t) P^-_t with P^-_t = d_t^2 P_{t-1} + 1
//     and K_t = lambda P^-_t / (lambda P^-_t + 1) is a linear-fractional map of
//     P_{t-1}, i.e. a 2x2 matrix on (P, 1) (composed with rescaling, since only
//     ratios matter): k_elk_riccati + k_elk_riccati_carry;
//  2. the filter mean m_t = (1 - K_t)(d_t m_{t-1} + r_t), an affine scan:
//     k_elk_mean + k_elk_mean_carry;
//  3. the Rauch-Tung-Striebel smoother m^s_t = G_t m^s_{t+1} + e_t with
//     G_t = P_t d_{t+1} / P^-_{t+1}, e_t = m_t - G_t (d_{t+1} m_t + r_{t+1}), a
//     reverse affine scan: k_elk_gains (stores G, e and each chunk's reverse
//     aggregate) + k_elk_smooth_carry, then k_elk_apply walks each chunk back
//     from its carry, h += m^s, and measures max |m^s|.
// lambda = 0 gives K = 0 and the quasi-DEER step.
#include <algorithm>

#include "cells_chan.h"
#include "internal.h"

namespace pr {

constexpr int ELK_L = 64;  // steps per chunk

int elk_chunk_len() { return ELK_L; }

struct ElkGeom {
  int b, j, t0, t1, i;  // sequence, chunk, its steps [t0, t1), this lane's state entry
  bool active;
};
__device__ inline ElkGeom elk_geom(const ElkArgs &a) {
  ElkGeom g;
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6), CG = (a.S + 63) / 64;
  const int cg = wave % CG, chunk = wave / CG;
  g.b = chunk / a.cps;
  g.j = chunk % a.cps;
  g.t0 = g.j * ELK_L;
  g.t1 = min(a.T, g.t0 + ELK_L);
  g.i = cg * 64 + (threadIdx.x & 63);
  g.active = chunk < a.nch && g.i < a.S;
  return g;
}

// 1. Riccati: each chunk's 2x2 map on (P, 1), [chunk][4][S]
__global__ __launch_bounds__(256) void k_elk_riccati(const ElkArgs a) {
  __shared__ int s_stop;
  if (sweep_is_stopped(a.st, &s_stop)) return;
  const ElkGeom g = elk_geom(a);
  if (!g.active) return;
  const int S = a.S;
  const float lam = a.lam;
  float m00 = 1.f, m01 = 0.f, m10 = 0.f, m11 = 1.f;
  for (int t = g.t0; t < g.t1; t++) {
    const float d = a.jr[((size_t)g.b * a.T + t) * 2 * S + g.i], d2 = d * d;
    // [[d^2, 1], [lambda d^2, lambda + 1]] applied after the maps so far
    const float n00 = d2 * m00 + m10, n01 = d2 * m01 + m11;
    const float n10 = lam * d2 * m00 + (lam + 1.f) * m10, n11 = lam * d2 * m01 + (lam + 1.f) * m11;
    const float sc = 1.f / fmaxf(fmaxf(n00, n01), fmaxf(n10, n11));  // entries are >= 0, n11 >= 1 before scaling
    m00 = n00 * sc; m01 = n01 * sc; m10 = n10 * sc; m11 = n11 * sc;
  }
  float *o = a.r1 + ((size_t)g.b * a.cps + g.j) * 4 * S + g.i;
  o[0] = m00; o[S] = m01; o[2 * S] = m10; o[3 * S] = m11;
}

// One wavefront per (sequence, entry); lanes take 64 chunks at a time.
__device__ inline bool elk_carry_geom(const ElkArgs &a, int &b, int &i) {
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
  b = w / a.S;
  i = w % a.S;
  return w < a.B * a.S;
}

// P entering each chunk, [chunk][S]
__global__ __launch_bounds__(256) void k_elk_riccati_carry(const ElkArgs a) {
  __shared__ int s_stop;
  if (sweep_is_stopped(a.st, &s_stop)) return;
  int b, i;
  if (!elk_carry_geom(a, b, i)) return;
  const int lane = threadIdx.x & 63, S = a.S, cps = a.cps;
  // running map applied to (0, 1): the state entering the current group
  float c0 = 0.f, c1 = 1.f;
  for (int g0 = 0; g0 < cps; g0 += 64) {
    const int jj = g0 + lane;
    const float *r = a.r1 + ((size_t)b * cps + min(jj, cps - 1)) * 4 * S + i;
    float m00 = r[0], m01 = r[S], m10 = r[2 * S], m11 = r[3 * S];
    if (jj >= cps) { m00 = 1.f; m01 = 0.f; m10 = 0.f; m11 = 1.f; }
    // inclusive scan: later maps applied after earlier ones
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float e00 = __shfl_up(m00, off, 64), e01 = __shfl_up(m01, off, 64);
      const float e10 = __shfl_up(m10, off, 64), e11 = __shfl_up(m11, off, 64);
      if (lane >= off) {
        const float n00 = m00 * e00 + m01 * e10, n01 = m00 * e01 + m01 * e11;
        const float n10 = m10 * e00 + m11 * e10, n11 = m10 * e01 + m11 * e11;
        const float sc = 1.f / fmaxf(fmaxf(n00, n01), fmaxf(n10, n11));
        m00 = n00 * sc; m01 = n01 * sc; m10 = n10 * sc; m11 = n11 * sc;
      }
    }
    // exclusive prefix applied to the running (c0, c1)
    const float p00 = __shfl_up(m00, 1, 64), p01 = __shfl_up(m01, 1, 64);
    const float p10 = __shfl_up(m10, 1, 64), p11 = __shfl_up(m11, 1, 64);
    const float u0 = lane == 0 ? c0 : p00 * c0 + p01 * c1, u1 = lane == 0 ? c1 : p10 * c0 + p11 * c1;
    if (jj < cps) a.pc[((size_t)b * cps + jj) * S + i] = u0 / u1;
    const float l00 = __shfl(m00, 63, 64), l01 = __shfl(m01, 63, 64), l10 = __shfl(m10, 63, 64),
                l11 = __shfl(m11, 63, 64);
    const float n0 = l00 * c0 + l01 * c1, n1 = l10 * c0 + l11 * c1;
    const float sc = 1.f / fmaxf(n0, n1);
    c0 = n0 * sc;
    c1 = n1 * sc;
  }
}

// 2. filter mean: each chunk's affine map m -> A m + B, [chunk][2][S]
__global__ __launch_bounds__(256) void k_elk_mean(const ElkArgs a) {
  __shared__ int s_stop;
  if (sweep_is_stopped(a.st, &s_stop)) return;
  const ElkGeom g = elk_geom(a);
  if (!g.active) return;
  const int S = a.S;
  const float lam = a.lam;
  float P = a.pc[((size_t)g.b * a.cps + g.j) * S + g.i], A = 1.f, Bv = 0.f;
  for (int t = g.t0; t < g.t1; t++) {
    const float *row = a.jr + ((size_t)g.b * a.T + t) * 2 * S;
    const float d = row[g.i], r = row[S + g.i];
    const float pp = fmaf(d * d, P, 1.f), k1 = 1.f / fmaf(lam, pp, 1.f);
    const float ca = k1 * d;
    Bv = fmaf(ca, Bv, k1 * r);
    A *= ca;
    P = k1 * pp;
  }
  float *o = a.r2 + ((size_t)g.b * a.cps + g.j) * 2 * S + g.i;
  o[0] = A;
  o[S] = Bv;
}

// affine scan over chunks (forward: state entering each chunk from 0;
// reverse: value entering each chunk from the right, 0 past the end)
template <bool REV>
__device__ inline void elk_affine_carry(const ElkArgs &a, const float *agg, float *out, int b, int i) {
  const int lane = threadIdx.x & 63, S = a.S, cps = a.cps;
  float c = 0.f;
  for (int g0 = 0; g0 < cps; g0 += 64) {
    const int q = g0 + lane;                   // position in scan order
    const int jj = REV ? cps - 1 - q : q;      // chunk
    const float *r = agg + ((size_t)b * cps + (q < cps ? jj : 0)) * 2 * S + i;
    float A = q < cps ? r[0] : 1.f, Bv = q < cps ? r[S] : 0.f;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float Ae = __shfl_up(A, off, 64), Be = __shfl_up(Bv, off, 64);
      if (lane >= off) {
        Bv = fmaf(A, Be, Bv);
        A *= Ae;
      }
    }
    const float Ai = __shfl_up(A, 1, 64), Bi = __shfl_up(Bv, 1, 64);
    if (q < cps) out[((size_t)b * cps + jj) * S + i] = lane == 0 ? c : fmaf(Ai, c, Bi);
    c = fmaf(__shfl(A, 63, 64), c, __shfl(Bv, 63, 64));
  }
}

__global__ __launch_bounds__(256) void k_elk_mean_carry(const ElkArgs a) {
  __shared__ int s_stop;
  if (sweep_is_stopped(a.st, &s_stop)) return;
  int b, i;
  if (!elk_carry_geom(a, b, i)) return;
  elk_affine_carry<false>(a, a.r2, a.mc, b, i);
}

// 3. smoother gains: G_t, e_t stored [row][G (S) | e (S)], and each chunk's
// reverse map m^s_{t0} = A m^s_{t1} + B, [chunk][2][S]
__global__ __launch_bounds__(256) void k_elk_gains(const ElkArgs a) {
  __shared__ int s_stop;
  if (sweep_is_stopped(a.st, &s_stop)) return;
  const ElkGeom g = elk_geom(a);
  if (!g.active) return;
  const int S = a.S, T = a.T;
  const float lam = a.lam;
  const size_t ch = (size_t)g.b * a.cps + g.j;
  float P = a.pc[ch * S + g.i], m = a.mc[ch * S + g.i];
  float Racc = 1.f, Sacc = 0.f;
  // filtered moments of step t, then the gain of step t from step t + 1's prediction
  const float *row = a.jr + ((size_t)g.b * T + g.t0) * 2 * S;
  float d = row[g.i], r = row[S + g.i];
  float pp = fmaf(d * d, P, 1.f), k1 = 1.f / fmaf(lam, pp, 1.f);
  P = k1 * pp;
  m = k1 * fmaf(d, m, r);
  for (int t = g.t0; t < g.t1; t++) {
    float G = 0.f, e = m;  // the sequence's last step: m^s = m
    float Pn = P, mn = m;
    if (t + 1 < T) {
      const float *rn = a.jr + ((size_t)g.b * T + t + 1) * 2 * S;
      const float dn = rn[g.i], rr = rn[S + g.i];
      const float ppn = fmaf(dn * dn, P, 1.f), mpn = fmaf(dn, m, rr);
      G = P * dn / ppn;
      e = fmaf(-G, mpn, m);
      const float kn = 1.f / fmaf(lam, ppn, 1.f);
      Pn = kn * ppn;
      mn = kn * mpn;
    }
    float *ge = a.ge + ((size_t)g.b * T + t) * 2 * S;
    ge[g.i] = G;
    ge[S + g.i] = e;
    Sacc = fmaf(Racc, e, Sacc);
    Racc *= G;
    P = Pn;
    m = mn;
  }
  float *o = a.r3 + ch * 2 * S + g.i;
  o[0] = Racc;
  o[S] = Sacc;
}

__global__ __launch_bounds__(256) void k_elk_smooth_carry(const ElkArgs a) {
  __shared__ int s_stop;
  if (sweep_is_stopped(a.st, &s_stop)) return;
  int b, i;
  if (!elk_carry_geom(a, b, i)) return;
  elk_affine_carry<true>(a, a.r3, a.msc, b, i);
}

// 4. smoother values from each chunk's right-hand carry, h += m^s, max |m^s|
template <typename ST>
__global__ __launch_bounds__(256) void k_elk_apply(const ElkArgs a) {
  __shared__ int s_stop;
  __shared__ unsigned s_dmax[4];
  if (sweep_is_stopped(a.st, &s_stop)) return;
  const ElkGeom g = elk_geom(a);
  const int S = a.S, T = a.T;
  const bool first = a.k == 1;  // the iterate is h = 0 before sweep 1
  unsigned dmax = 0;
  if (g.active) {
    float y = a.msc[((size_t)g.b * a.cps + g.j) * S + g.i];
    ST *h = (ST *)a.h;
    for (int t = g.t1 - 1; t >= g.t0; t--) {
      const size_t row = (size_t)g.b * T + t;
      const float *ge = a.ge + row * 2 * S;
      y = fmaf(ge[g.i], y, ge[S + g.i]);
      const float hv = first ? 0.f : ldf(h, row * S + g.i);
      if constexpr (sizeof(ST) == 2) h[row * S + g.i] = f2bf(hv + y);
      else h[row * S + g.i] = hv + y;
      const unsigned u = __float_as_uint(fabsf(y));
      dmax = u > dmax ? u : dmax;
    }
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

// Producer for the per-channel cells: the Jacobian's diagonal and the
// residual at the current iterate, one thread per (row, channel).
template <int CELL, typename ST>
__global__ __launch_bounds__(256) void k_elk_jr_chan(const ElkChanArgs a) {
  __shared__ int s_stop;
  if (sweep_open(a.e.st, a.e.k, a.e.tol, a.e.T, a.e.max_iters, &s_stop)) return;
  constexpr int SW = cell_code(CELL) == C_LSTM ? 2 : 1;
  const int n = a.n, S = a.e.S, T = a.e.T;
  const size_t rows = (size_t)a.e.B * T;
  const bool first = a.e.k == 1;
  for (size_t e = (size_t)blockIdx.x * 256 + threadIdx.x; e < rows * n; e += (size_t)gridDim.x * 256) {
    const size_t row = e / n;
    const int c = (int)(e % n), t = (int)(row % T), b = (int)(row / T);
    const ST *Wh = (const ST *)a.Wh, *bh = (const ST *)a.bh, *pe = (const ST *)a.peep;
    ChanW w;
    w.a0 = ldf(Wh, c); w.a1 = ldf(Wh, (size_t)n + c); w.a2 = ldf(Wh, (size_t)2 * n + c);
    w.b0 = bh ? ldf(bh, c) : 0.f; w.b1 = bh ? ldf(bh, (size_t)n + c) : 0.f; w.b2 = bh ? ldf(bh, (size_t)2 * n + c) : 0.f;
    w.p0 = pe ? ldf(pe, c) : 0.f; w.p1 = pe ? ldf(pe, (size_t)n + c) : 0.f;
    const ST *U = (const ST *)a.U + row * 3 * n;
    const float u[3] = {ldf(U, c), ldf(U, (size_t)n + c), ldf(U, (size_t)2 * n + c)};
    float s[SW], hc[SW];
#pragma unroll
    for (int q = 0; q < SW; q++) {
      const int idx = c * SW + q;
      float sv = 0.f;
      if (t > 0) sv = first ? 0.f : ldf((const ST *)a.e.h, (row - 1) * S + idx);
      else if (a.h0) sv = ldf((const ST *)a.h0, (size_t)b * S + idx);
      s[q] = sv;
      hc[q] = first ? 0.f : ldf((const ST *)a.e.h, row * S + idx);
    }
    float f[SW], J[SW * SW];
    chan_cell<CELL>(s, u, w, f, J);
    float *out = a.e.jr + row * 2 * S;
#pragma unroll
    for (int q = 0; q < SW; q++) {
      out[c * SW + q] = J[q * SW + q];
      out[S + c * SW + q] = f[q] - hc[q];
    }
  }
}

hipError_t launch_elk_sweep(ElkArgs &a, hipStream_t s) {
  const int CG = (a.S + 63) / 64;
  const unsigned gchunks = (unsigned)(((size_t)a.nch * CG + 3) / 4);
  const unsigned gcarry = (unsigned)(((size_t)a.B * a.S + 3) / 4);
  hipLaunchKernelGGL(k_elk_riccati, dim3(gchunks), dim3(256), 0, s, a);
  hipLaunchKernelGGL(k_elk_riccati_carry, dim3(gcarry), dim3(256), 0, s, a);
  hipLaunchKernelGGL(k_elk_mean, dim3(gchunks), dim3(256), 0, s, a);
  hipLaunchKernelGGL(k_elk_mean_carry, dim3(gcarry), dim3(256), 0, s, a);
  hipLaunchKernelGGL(k_elk_gains, dim3(gchunks), dim3(256), 0, s, a);
  hipLaunchKernelGGL(k_elk_smooth_carry, dim3(gcarry), dim3(256), 0, s, a);
  if (a.h_bf16) hipLaunchKernelGGL(k_elk_apply<uint16_t>, dim3(gchunks), dim3(256), 0, s, a);
  else hipLaunchKernelGGL(k_elk_apply<float>, dim3(gchunks), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_elk_jr_chan(int cell, bool bf16, const ElkChanArgs &a, hipStream_t s) {
  const size_t work = (size_t)a.e.B * a.e.T * a.n;
  const unsigned grid = (unsigned)std::min<size_t>((work + 255) / 256, 65536);
  if (cell == C_GRU_DIAG) {
    if (bf16) hipLaunchKernelGGL((k_elk_jr_chan<C_GRU_DIAG, uint16_t>), dim3(grid), dim3(256), 0, s, a);
    else hipLaunchKernelGGL((k_elk_jr_chan<C_GRU_DIAG, float>), dim3(grid), dim3(256), 0, s, a);
  } else {
    constexpr int C = C_LSTM + 16 * APX_DIAG;
    if (bf16) hipLaunchKernelGGL((k_elk_jr_chan<C, uint16_t>), dim3(grid), dim3(256), 0, s, a);
    else hipLaunchKernelGGL((k_elk_jr_chan<C, float>), dim3(grid), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace pr

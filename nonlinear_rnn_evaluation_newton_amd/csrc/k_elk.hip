// Quasi-ELK sweeps: the Levenberg-Marquardt-damped quasi-Newton step solved
// as a Kalman smoother (Gonzalez et al. abstract: ELK stabilises DEER through
// the connection between Levenberg-Marquardt and Kalman smoothing; Para-Seq
// README, Main features: ELK and quasi-ELK solvers).
//
// With the Jacobian's diagonal d_t, every state entry i is a scalar model
//   dh_t = d_t dh_{t-1} + r_t + w_t,  w_t ~ N(0, 1),   0 = dh_t + v_t,
//   v_t ~ N(0, 1 / lambda),   dh_{-1} = 0,
// whose posterior mean is the damped step argmin ||L dh - r||^2 + lambda ||dh||^2.
// The filter, P_t = (1 - K_t) P^-_t and m_t = (1 - K_t)(d_t m_{t-1} + r_t) with
// P^-_t = d_t^2 P_{t-1} + 1 and K_t = lambda P^-_t / (lambda P^-_t + 1), is
// one linear scan in homogeneous coordinates (H7 below); the
// Rauch-Tung-Striebel smoother m^s_t = G_t m^s_{t+1} + e_t with
// G_t = P_t d_{t+1} / P^-_{t+1} and e_t = m_t - G_t (d_{t+1} m_t + r_{t+1}) is a
// reverse affine scan.
//
// Dense n = 64 GRU: the gates kernel has stored d_t and r_t at the current
// iterate ([row][d (S) | r (S)], fp32); a lane per (chunk, state entry), a
// wavefront per 64 entries of a chunk or per 64 / sp chunks of sp entries:
//   k_elk_filter + k_elk_filter_carry   chunk filter maps, moments entering
//                                       each chunk (shuffle scan over chunks);
//   k_elk_gains + k_elk_smooth_carry    G, e per step and each chunk's
//                                       reverse map, m^s entering from the right;
//   k_elk_apply                         each chunk walked back from its carry,
//                                       h += m^s, max |m^s|.
// Per-channel cells: further below.
// lambda = 0 gives K = 0 and the quasi-DEER step.
#include <algorithm>

#include "k_chan_impl.h"
#include "internal.h"

namespace pr {

// Lanes per chunk (the state width rounded up to a power of two, at most 64)
// and steps per chunk.  A narrow state packs 64 / sp chunks into a
// wavefront, and takes longer chunks so the serial walks over chunk
// aggregates stay short.
static int elk_lanes(int S) {
  int sp = 1;
  while (sp < S && sp < 64) sp *= 2;
  return sp;
}
int elk_chunk_len(int S) {
  const int sp = elk_lanes(S);
  return sp >= 4 ? 64 : 256 / sp;
}
int elk_lanes_per_chunk(int S) { return elk_lanes(S); }

struct ElkGeom {
  int b, j, t0, t1, i;  // sequence, chunk, its steps [t0, t1), this lane's state entry
  bool active;
};
__device__ inline ElkGeom elk_geom(const ElkArgs &a) {
  ElkGeom g;
  const int lane = threadIdx.x & 63, sp = a.sp;
  const int wave = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6), CG = (a.S + sp - 1) / sp;
  const int cg = wave % CG, chunk = (wave / CG) * (64 / sp) + lane / sp;
  g.b = chunk / a.cps;
  g.j = chunk % a.cps;
  g.t0 = g.j * a.L;
  g.t1 = min(a.T, g.t0 + a.L);
  g.i = cg * sp + lane % sp;
  g.active = chunk < a.nch && g.i < a.S;
  return g;
}

// Homogeneous filter map [[a, 0, b], [c, e, f], [g, 0, h]] on (p, mu, q) with
// P = p / q and m = mu / q; one step is
//   p' = d^2 p + q,  mu' = d mu + r q,  q' = lambda d^2 p + (lambda + 1) q.
struct H7 {
  float a, b, c, e, f, g, h;
};
__device__ inline void h7_scale(H7 &m) {
  const float s = frcp(fmaxf(fmaxf(m.a, m.b), fmaxf(m.g, m.h)));  // any positive factor works
  m.a *= s; m.b *= s; m.c *= s; m.e *= s; m.f *= s; m.g *= s; m.h *= s;
}
__device__ inline H7 h7_id() { return H7{1.f, 0.f, 0.f, 1.f, 0.f, 0.f, 1.f}; }
// X applied after Y
__device__ inline H7 h7_after(const H7 &X, const H7 &Y) {
  H7 o;
  o.a = fmaf(X.a, Y.a, X.b * Y.g);
  o.b = fmaf(X.a, Y.b, X.b * Y.h);
  o.g = fmaf(X.g, Y.a, X.h * Y.g);
  o.h = fmaf(X.g, Y.b, X.h * Y.h);
  o.e = X.e * Y.e;
  o.c = fmaf(X.c, Y.a, fmaf(X.e, Y.c, X.f * Y.g));
  o.f = fmaf(X.c, Y.b, fmaf(X.e, Y.f, X.f * Y.h));
  h7_scale(o);
  return o;
}
__device__ inline H7 h7_shfl_up(const H7 &M, int off) {
  return H7{__shfl_up(M.a, off, 64), __shfl_up(M.b, off, 64), __shfl_up(M.c, off, 64), __shfl_up(M.e, off, 64),
            __shfl_up(M.f, off, 64), __shfl_up(M.g, off, 64), __shfl_up(M.h, off, 64)};
}
__device__ inline H7 h7_shfl(const H7 &M, int lane) {
  return H7{__shfl(M.a, lane, 64), __shfl(M.b, lane, 64), __shfl(M.c, lane, 64), __shfl(M.e, lane, 64),
            __shfl(M.f, lane, 64), __shfl(M.g, lane, 64), __shfl(M.h, lane, 64)};
}
// one step (d, r) applied after m
__device__ inline void h7_step(H7 &m, float d, float r, float lam, float lam1) {
  const float d2 = d * d, ld2 = lam * d2;
  H7 o;
  o.a = fmaf(d2, m.a, m.g);
  o.b = fmaf(d2, m.b, m.h);
  o.c = fmaf(d, m.c, r * m.g);
  o.e = d * m.e;
  o.f = fmaf(d, m.f, r * m.h);
  o.g = fmaf(ld2, m.a, lam1 * m.g);
  o.h = fmaf(ld2, m.b, lam1 * m.h);
  h7_scale(o);
  m = o;
}

// 1. filter: each chunk's homogeneous filter map (seven numbers, as for the
// per-channel cells below), [chunk][7][S]
__global__ __launch_bounds__(256) void k_elk_filter(const ElkArgs a) {
  __shared__ int s_stop;
  if (sweep_is_stopped(a.st, &s_stop)) return;
  const ElkGeom g = elk_geom(a);
  if (!g.active) return;
  const int S = a.S;
  const float lam = a.lam, lam1 = lam + 1.f;
  H7 m = h7_id();
  for (int t = g.t0; t < g.t1; t++) {
    const float *row = a.jr + ((size_t)g.b * a.T + t) * 2 * S;
    h7_step(m, row[g.i], row[S + g.i], lam, lam1);
  }
  float *o = a.r1 + ((size_t)g.b * a.cps + g.j) * 7 * S + g.i;
  o[0] = m.a; o[S] = m.b; o[2 * S] = m.c; o[3 * S] = m.e; o[4 * S] = m.f; o[5 * S] = m.g; o[6 * S] = m.h;
}

// One wavefront per (sequence, entry); lanes take 64 chunks at a time.
__device__ inline bool elk_carry_geom(const ElkArgs &a, int &b, int &i) {
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
  b = w / a.S;
  i = w % a.S;
  return w < a.B * a.S;
}

// filtered moments (P, m) entering each chunk, [chunk][S] each: the chunk
// maps composed by a shuffle scan, 64 chunks at a time
__global__ __launch_bounds__(256) void k_elk_filter_carry(const ElkArgs a) {
  __shared__ int s_stop;
  if (sweep_is_stopped(a.st, &s_stop)) return;
  int b, i;
  if (!elk_carry_geom(a, b, i)) return;
  const int lane = threadIdx.x & 63, S = a.S, cps = a.cps;
  float cp = 0.f, cm = 0.f;  // running (P, m); dh_{-1} = 0 is known exactly
  for (int g0 = 0; g0 < cps; g0 += 64) {
    const int jj = g0 + lane;
    H7 M = h7_id();
    if (jj < cps) {
      const float *r = a.r1 + ((size_t)b * cps + jj) * 7 * S + i;
      M = H7{r[0], r[S], r[2 * S], r[3 * S], r[4 * S], r[5 * S], r[6 * S]};
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const H7 E = h7_shfl_up(M, off);
      if (lane >= off) M = h7_after(M, E);
    }
    H7 E = h7_shfl_up(M, 1);
    if (lane == 0) E = h7_id();
    if (jj < cps) {
      const float p = fmaf(E.a, cp, E.b), mu = fmaf(E.c, cp, fmaf(E.e, cm, E.f)), q = fmaf(E.g, cp, E.h);
      a.pc[((size_t)b * cps + jj) * S + i] = p / q;
      a.mc[((size_t)b * cps + jj) * S + i] = mu / q;
    }
    const H7 L = h7_shfl(M, 63);
    const float p = fmaf(L.a, cp, L.b), mu = fmaf(L.c, cp, fmaf(L.e, cm, L.f)), q = fmaf(L.g, cp, L.h);
    cp = p / q;
    cm = mu / q;
  }
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
  float pp = fmaf(d * d, P, 1.f), k1 = frcp(fmaf(lam, pp, 1.f));
  P = k1 * pp;
  m = k1 * fmaf(d, m, r);
  for (int t = g.t0; t < g.t1; t++) {
    float G = 0.f, e = m;  // the sequence's last step: m^s = m
    float Pn = P, mn = m;
    if (t + 1 < T) {
      const float *rn = a.jr + ((size_t)g.b * T + t + 1) * 2 * S;
      const float dn = rn[g.i], rr = rn[S + g.i];
      const float ppn = fmaf(dn * dn, P, 1.f), mpn = fmaf(dn, m, rr);
      G = P * dn * frcp(ppn);
      e = fmaf(-G, mpn, m);
      const float kn = frcp(fmaf(lam, ppn, 1.f));
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

// ---------------------------------------------------------------------------
// Per-channel cells: the sweep re-evaluates the cell in each of its three
// passes instead of storing d_t and r_t (the inputs, U and the iterate, cost
// fewer bytes per step than [d | r] in fp32 and are read, not written).
//
// The filter is one linear scan in homogeneous coordinates: with P = p / q
// and m = mu / q, one step is the 3x3 map
//   p' = d^2 p + q,  mu' = d mu + r q,  q' = lambda d^2 p + (lambda + 1) q,
// whose products keep the zero pattern [[a, 0, b], [c, e, f], [g, 0, h]]
// (seven numbers, rescaled freely since only ratios matter).  The filter and
// smoother passes walk chunks of ELKC_SUB * L steps; the apply pass, which
// keeps a chunk's gains in registers, walks chunks of L.  Per sweep:
//   k_elkc_filter        each chunk's filter map          [chunk][7][S]
//   k_elkc_filter_carry  (P, m) entering each chunk       [chunk][2][S]
//   k_elkc_smooth        filter from the carry and smoother gains; per apply
//                        chunk: (P, m) entering it, its reverse map (R, S),
//                        and what the apply pass needs from its neighbours'
//                        rows, which that pass overwrites: d, r of the next
//                        chunk's first step and the state at its last step
//   k_elkc_smooth_carry  m^s entering each filter chunk from the right (the
//                        apply pass carries it through the later apply chunks)
//   k_elkc_apply         filter and gains again (kept in registers), then the
//                        chunk walked backwards: h += m^s, max |m^s|
// One wavefront per (sequence, chunk, 64 channels); a lane owns one channel
// and its SW state entries.
// ---------------------------------------------------------------------------


template <int CELL>
constexpr int elkc_sw() {
  return cell_code(CELL) == C_LSTM ? 2 : 1;
}
template <int CELL>
constexpr int elkc_len() {
  return elkc_sw<CELL>() == 1 ? 32 : 16;  // the apply pass keeps 2 * SW * L gains in registers
}
constexpr int ELKC_SUB = 4;  // apply chunks per filter / smoother chunk
int elk_chan_chunk_len(int sw) { return sw == 1 ? 32 : 16; }

struct ElkcGeom {
  int b, j, t0, t1, c;  // sequence, chunk, its steps [t0, t1), channel (clamped to n - 1)
  size_t ch;            // chunk index over all sequences
  bool wave_on, on;     // the wavefront has a chunk; this lane has a channel
};
template <int LC>
__device__ inline ElkcGeom elkc_geom(const ElkChanArgs &a, int cps, int nch) {
  ElkcGeom g;
  // wave-uniform, so the chunk's buffer resources live in scalar registers
  const int wave = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6), CG = (a.n + 63) / 64;
  const int cg = wave % CG, chunk = wave / CG;
  g.wave_on = chunk < nch;
  g.ch = (size_t)min(chunk, nch - 1);
  g.b = (int)(g.ch / cps);
  g.j = (int)(g.ch % cps);
  g.t0 = g.j * LC;
  g.t1 = min(a.e.T, g.t0 + LC);
  const int c = cg * 64 + (threadIdx.x & 63);
  g.on = g.wave_on && c < a.n;
  g.c = min(c, a.n - 1);
  return g;
}

template <typename ST, int CELL>
__device__ inline ChanW elkc_weights(const ElkChanArgs &a, int c) {
  const int n = a.n;
  const ST *Wh = (const ST *)a.Wh, *bh = (const ST *)a.bh, *pe = (const ST *)a.peep;
  ChanW w;
  w.a0 = ldf(Wh, c); w.a1 = ldf(Wh, (size_t)n + c); w.a2 = ldf(Wh, (size_t)2 * n + c);
  w.b0 = bh ? ldf(bh, c) : 0.f; w.b1 = bh ? ldf(bh, (size_t)n + c) : 0.f; w.b2 = bh ? ldf(bh, (size_t)2 * n + c) : 0.f;
  w.p0 = pe ? ldf(pe, c) : 0.f; w.p1 = pe ? ldf(pe, (size_t)n + c) : 0.f;
  chan_w_scale<CELL>(w);
  return w;
}

// the iterate's entries of channel c at step t (0 before sweep 1)
template <typename ST, int SW>
__device__ inline void elkc_ld_h(const ElkChanArgs &a, bool first, size_t row, int c, float *o) {
  if (first) {
#pragma unroll
    for (int q = 0; q < SW; q++) o[q] = 0.f;
  } else {
    ld_vec<ST, SW>((const ST *)a.e.h + row * a.e.S + (size_t)c * SW, o);
  }
}

// the initial state's entries of sequence b (0 without one)
template <typename ST, int SW>
__device__ inline void elkc_ld_h0(const ElkChanArgs &a, int b, int c, float *o) {
#pragma unroll
  for (int q = 0; q < SW; q++) o[q] = a.h0 ? ldf((const ST *)a.h0, (size_t)b * a.e.S + (size_t)c * SW + q) : 0.f;
}

// CNT values of storage type ST at byte offset off of r (0 past its end)
template <typename ST, int CNT>
__device__ inline void elkc_bld(Rsrc r, unsigned off, float *o) {
  unsigned w[words_of<ST, CNT>()];
  bldw<CNT * (int)sizeof(ST)>(r, off, w);
#pragma unroll
  for (int q = 0; q < CNT; q++) o[q] = unpackw<ST>(w, q);
}

// Buffer resources over the chunk's rows of U and of the iterate: offsets
// stay 32-bit and small, and rows past the chunk read 0.
struct ElkcRows {
  Rsrc U, H;
};
template <typename ST>
__device__ inline ElkcRows elkc_rows(const ElkChanArgs &a, const ElkcGeom &g, int t0, int nrows) {
  const size_t row0 = (size_t)g.b * a.e.T + t0;
  ElkcRows r;
  r.U = sc_rsrc((const ST *)a.U + row0 * 3 * a.n, (unsigned)(nrows * 3 * a.n * (int)sizeof(ST)));
  r.H = sc_rsrc((const ST *)a.e.h + row0 * a.e.S, (unsigned)(nrows * a.e.S * (int)sizeof(ST)));
  return r;
}

// U (3 gates) and the iterate (SW values, 0 before sweep 1) of channel c at
// row i of a chunk's resources
template <typename ST, int SW>
__device__ inline void elkc_ld_step(const ElkcRows &rs, const ElkChanArgs &a, int c, bool first, int i, float *u,
                                    float *hc) {
  const unsigned ub = (unsigned)(i * 3 * a.n + c) * (unsigned)sizeof(ST);
#pragma unroll
  for (int q = 0; q < 3; q++) elkc_bld<ST, 1>(rs.U, ub + (unsigned)(q * a.n) * (unsigned)sizeof(ST), u + q);
  if (first) {
#pragma unroll
    for (int q = 0; q < SW; q++) hc[q] = 0.f;
  } else {
    elkc_bld<ST, SW>(rs.H, (unsigned)(i * a.e.S + c * SW) * (unsigned)sizeof(ST), hc);
  }
}

// d and r of every step of the chunk, in order: fn(i, d, r) with s the
// iterate at step i - 1 (the state before t0 for i = 0); s leaves as the
// iterate at t1 - 1.  Loads run one group
// of 8 steps ahead.
template <int CELL, typename ST, int LC, typename F>
__device__ inline void elkc_walk(const ElkChanArgs &a, const ElkcGeom &g, const ChanW &w, bool first, float *s, F &&fn) {
  constexpr int SW = elkc_sw<CELL>(), P = 8, NG = LC / P;
  const ElkcRows rs = elkc_rows<ST>(a, g, g.t0, g.t1 - g.t0);
  float u[2][P][3], hc[2][P][SW];
  auto load = [&](int grp, int buf) {
#pragma unroll
    for (int p = 0; p < P; p++) elkc_ld_step<ST, SW>(rs, a, g.c, first, grp * P + p, u[buf][p], hc[buf][p]);
  };
  load(0, 0);
#pragma unroll
  for (int grp = 0; grp < NG; grp++) {
    if (grp + 1 < NG) load(grp + 1, (grp + 1) & 1);
#pragma unroll
    for (int p = 0; p < P; p++) {
      const int i = grp * P + p;
      if (g.t0 + i < g.t1) {
        float f[SW], J[SW * SW], d[SW], r[SW];
        chan_cell<CELL>(s, u[grp & 1][p], w, f, J);
#pragma unroll
        for (int q = 0; q < SW; q++) {
          d[q] = J[q * SW + q];
          r[q] = f[q] - hc[grp & 1][p][q];
        }
        fn(i, d, r);
#pragma unroll
        for (int q = 0; q < SW; q++) s[q] = hc[grp & 1][p][q];
      }
    }
  }
}

// d and r at step t1 (the next chunk's first step), from the iterate at
// t1 - 1 (s) and t1
template <int CELL, typename ST>
__device__ inline void elkc_next(const ElkChanArgs &a, const ElkcGeom &g, const ChanW &w, bool first, const float *s,
                                 float *d, float *r) {
  constexpr int SW = elkc_sw<CELL>();
  const ElkcRows rs = elkc_rows<ST>(a, g, g.t1, 1);
  float u[3], hc[SW], f[SW], J[SW * SW];
  elkc_ld_step<ST, SW>(rs, a, g.c, first, 0, u, hc);
  chan_cell<CELL>(s, u, w, f, J);
#pragma unroll
  for (int q = 0; q < SW; q++) {
    d[q] = J[q * SW + q];
    r[q] = f[q] - hc[q];
  }
}

template <int CELL, typename ST>
__global__ __launch_bounds__(256) void k_elkc_filter(const ElkChanArgs a) {
  __shared__ int s_stop;
  if (sweep_open(a.e.st, a.e.k, a.e.tol, a.e.T, a.e.max_iters, &s_stop)) return;
  constexpr int SW = elkc_sw<CELL>(), LF = ELKC_SUB * elkc_len<CELL>();
  const ElkcGeom g = elkc_geom<LF>(a, a.cpf, a.nchf);
  if (!g.wave_on) return;
  const bool first = a.e.k == 1;
  const float lam = a.e.lam, lam1 = lam + 1.f;
  const ChanW w = elkc_weights<ST, CELL>(a, g.c);
  float s[SW];
  if (g.t0 == 0) elkc_ld_h0<ST, SW>(a, g.b, g.c, s);
  else elkc_ld_h<ST, SW>(a, first, (size_t)g.b * a.e.T + g.t0 - 1, g.c, s);
  H7 m[SW];
#pragma unroll
  for (int q = 0; q < SW; q++) m[q] = h7_id();
  elkc_walk<CELL, ST, LF>(a, g, w, first, s, [&](int, const float *d, const float *r) {
#pragma unroll
    for (int q = 0; q < SW; q++) h7_step(m[q], d[q], r[q], lam, lam1);
  });
  if (!g.on) return;
  const int S = a.e.S;
#pragma unroll
  for (int q = 0; q < SW; q++) {
    float *o = a.fagg + g.ch * 7 * S + (size_t)g.c * SW + q;
    o[0] = m[q].a; o[S] = m[q].b; o[2 * S] = m[q].c; o[3 * S] = m[q].e;
    o[4 * S] = m[q].f; o[5 * S] = m[q].g; o[6 * S] = m[q].h;
  }
}

// Chunk carries: a lane owns one (sequence, state entry), so a wavefront's
// loads of a chunk's aggregate are coalesced across 64 adjacent entries, and
// walks the chunks serially; loads run a batch of ELKC_CB chunks ahead of the
// composition.  One wavefront per block spreads the few wavefronts over all
// compute units.
constexpr int ELKC_CB = 8;

__device__ inline bool elkc_carry_lane(const ElkArgs &a, int &b, int &i) {
  const int e = blockIdx.x * 64 + (int)threadIdx.x;
  b = e / a.S;
  i = e % a.S;
  return e < a.B * a.S;
}

// (P, m) entering each chunk, [chunk][2][S]
__global__ __launch_bounds__(64) void k_elkc_filter_carry(const ElkChanArgs ca) {
  const ElkArgs &a = ca.e;
  __shared__ int s_stop;
  if (sweep_is_stopped(a.st, &s_stop)) return;
  int b, i;
  if (!elkc_carry_lane(a, b, i)) return;
  const int S = a.S, cps = ca.cpf;
  const float *src = ca.fagg + (size_t)b * cps * 7 * S + i;
  float *dst = ca.fcar + (size_t)b * cps * 2 * S + i;
  float cp = 0.f, cm = 0.f;  // running (P, m); dh_{-1} = 0 is known exactly
  float buf[2][ELKC_CB][7];
  auto load = [&](int j0, int k) {
#pragma unroll
    for (int c = 0; c < ELKC_CB; c++) {
      const float *r = src + (size_t)min(j0 + c, cps - 1) * 7 * S;
#pragma unroll
      for (int v = 0; v < 7; v++) buf[k][c][v] = r[(size_t)v * S];
    }
  };
  load(0, 0);
  for (int j0 = 0; j0 < cps; j0 += 2 * ELKC_CB) {
#pragma unroll
    for (int half = 0; half < 2; half++) {
      const int jb = j0 + half * ELKC_CB;
      if (jb >= cps) break;
      if (jb + ELKC_CB < cps) load(jb + ELKC_CB, half ^ 1);
#pragma unroll
      for (int c = 0; c < ELKC_CB; c++) {
        if (jb + c < cps) {
          float *o = dst + (size_t)(jb + c) * 2 * S;
          o[0] = cp;
          o[S] = cm;
          const float *M = buf[half][c];
          const float p = fmaf(M[0], cp, M[1]), mu = fmaf(M[2], cp, fmaf(M[3], cm, M[4])), q = fmaf(M[5], cp, M[6]);
          const float iq = 1.f / q;
          cp = p * iq;
          cm = mu * iq;
        }
      }
    }
  }
}

// m^s entering each filter chunk from the right (0 past the sequence's end),
// [chunk][S] in the filter carries' space, from the filter chunks' reverse
// maps (R, S) that the smoother pass left in the filter maps' space
__global__ __launch_bounds__(64) void k_elkc_smooth_carry(const ElkChanArgs ca) {
  const ElkArgs &a = ca.e;
  __shared__ int s_stop;
  if (sweep_is_stopped(a.st, &s_stop)) return;
  int b, i;
  if (!elkc_carry_lane(a, b, i)) return;
  const int S = a.S, cps = ca.cpf;
  const float *src = ca.fagg + (size_t)b * cps * 2 * S + i;
  float *dst = ca.fcar + (size_t)b * cps * S + i;
  float y = 0.f;
  float buf[2][ELKC_CB][2];
  auto load = [&](int q0, int k) {  // q counts chunks from the right
#pragma unroll
    for (int c = 0; c < ELKC_CB; c++) {
      const float *r = src + (size_t)max(cps - 1 - (q0 + c), 0) * 2 * S;
      buf[k][c][0] = r[0];
      buf[k][c][1] = r[S];
    }
  };
  load(0, 0);
  for (int q0 = 0; q0 < cps; q0 += 2 * ELKC_CB) {
#pragma unroll
    for (int half = 0; half < 2; half++) {
      const int qb = q0 + half * ELKC_CB;
      if (qb >= cps) break;
      if (qb + ELKC_CB < cps) load(qb + ELKC_CB, half ^ 1);
#pragma unroll
      for (int c = 0; c < ELKC_CB; c++) {
        if (qb + c < cps) {
          dst[(size_t)(cps - 1 - (qb + c)) * S] = y;
          y = fmaf(buf[half][c][0], y, buf[half][c][1]);
        }
      }
    }
  }
}

// smoother gains from the filter: G_t = P_t d_{t+1} / P^-_{t+1} and
// e_t = m_t - G_t (d_{t+1} m_t + r_{t+1}); at the sequence's last step G = 0
// and e = m.  (P, m) enter as the filtered moments before t0; fn(i, q, G, e)
// per entry, in step order.  The last step takes d, r of step t1 from the
// smoother pass's store.
template <int CELL, typename ST, int LC, typename F>
__device__ inline void elkc_gains(const ElkChanArgs &a, const ElkcGeom &g, const ChanW &w, bool first, float *s,
                                  float *P, float *m, F &&fn) {
  constexpr int SW = elkc_sw<CELL>();
  const float lam = a.e.lam;
  const int S = a.e.S;
  elkc_walk<CELL, ST, LC>(a, g, w, first, s, [&](int i, const float *d, const float *r) {
#pragma unroll
    for (int q = 0; q < SW; q++) {
      const float pp = fmaf(d[q] * d[q], P[q], 1.f), mp = fmaf(d[q], m[q], r[q]);
      if (i > 0) {
        const float G = P[q] * d[q] * frcp(pp);
        fn(i - 1, q, G, fmaf(-G, mp, m[q]));
      }
      const float k1 = frcp(fmaf(lam, pp, 1.f));
      P[q] = k1 * pp;
      m[q] = k1 * mp;
    }
  });
  const bool more = g.t1 < a.e.T;
  const int il = g.t1 - 1 - g.t0;
#pragma unroll
  for (int q = 0; q < SW; q++) {
    float G = 0.f, e = m[q];
    if (more) {
      const float *x = a.dr + g.ch * 2 * S + (size_t)g.c * SW + q;
      const float dn = x[0], rn = x[S];
      const float pp = fmaf(dn * dn, P[q], 1.f);
      G = P[q] * dn * frcp(pp);
      e = fmaf(-G, fmaf(dn, m[q], rn), m[q]);
    }
    fn(il, q, G, e);
  }
}

// Smoother pass over filter chunks of ELKC_SUB apply chunks: per apply chunk
// the filtered moments entering it, its reverse map m^s_{t0} = R m^s_{t1} + Sa
// (composed in step order), d, r at the step after it and the iterate at its
// last step.
template <int CELL, typename ST>
__global__ __launch_bounds__(256) void k_elkc_smooth(const ElkChanArgs a) {
  __shared__ int s_stop;
  if (sweep_is_stopped(a.e.st, &s_stop)) return;
  constexpr int SW = elkc_sw<CELL>(), LC = elkc_len<CELL>(), LF = ELKC_SUB * LC;
  const ElkcGeom g = elkc_geom<LF>(a, a.cpf, a.nchf);
  if (!g.wave_on) return;
  const bool first = a.e.k == 1;
  const int S = a.e.S;
  const float lam = a.e.lam;
  const size_t sub0 = (size_t)g.b * a.e.cps + (size_t)g.j * ELKC_SUB, col = (size_t)g.c * SW;
  const ChanW w = elkc_weights<ST, CELL>(a, g.c);
  float s[SW], P[SW], m[SW], R[SW], Sa[SW], RF[SW], SF[SW];
  if (g.t0 == 0) elkc_ld_h0<ST, SW>(a, g.b, g.c, s);
  else elkc_ld_h<ST, SW>(a, first, (size_t)g.b * a.e.T + g.t0 - 1, g.c, s);
#pragma unroll
  for (int q = 0; q < SW; q++) {
    const float *x = a.fcar + g.ch * 2 * S + col + q;
    P[q] = x[0];
    m[q] = x[S];
    R[q] = 1.f;
    Sa[q] = 0.f;
    RF[q] = 1.f;
    SF[q] = 0.f;
  }
  auto put_moments = [&](size_t sub) {
    if (!g.on) return;
#pragma unroll
    for (int q = 0; q < SW; q++) {
      a.fsub[sub * 2 * S + col + q] = P[q];
      a.fsub[sub * 2 * S + S + col + q] = m[q];
    }
  };
  auto put_chunk = [&](size_t sub, const float *dn, const float *rn, const float *hl) {
#pragma unroll
    for (int q = 0; q < SW; q++) {  // the filter chunk's reverse map, composed in step order
      SF[q] = fmaf(RF[q], Sa[q], SF[q]);
      RF[q] *= R[q];
    }
    if (!g.on) return;
#pragma unroll
    for (int q = 0; q < SW; q++) {
      a.e.r3[sub * 2 * S + col + q] = R[q];
      a.e.r3[sub * 2 * S + S + col + q] = Sa[q];
      a.dr[sub * 2 * S + col + q] = dn[q];
      a.dr[sub * 2 * S + S + col + q] = rn[q];
      a.hb[sub * S + col + q] = hl[q];
    }
  };
  put_moments(sub0);
  elkc_walk<CELL, ST, LF>(a, g, w, first, s, [&](int i, const float *d, const float *r) {
    float pp[SW], mp[SW];
#pragma unroll
    for (int q = 0; q < SW; q++) {
      pp[q] = fmaf(d[q] * d[q], P[q], 1.f);
      mp[q] = fmaf(d[q], m[q], r[q]);
      if (i > 0) {  // the gain of step i - 1
        const float G = P[q] * d[q] * frcp(pp[q]), e = fmaf(-G, mp[q], m[q]);
        Sa[q] = fmaf(R[q], e, Sa[q]);
        R[q] *= G;
      }
    }
    if (i > 0 && i % LC == 0) {  // step i - 1 closed an apply chunk; s is its last state
      put_chunk(sub0 + i / LC - 1, d, r, s);
#pragma unroll
      for (int q = 0; q < SW; q++) {
        R[q] = 1.f;
        Sa[q] = 0.f;
      }
      put_moments(sub0 + i / LC);
    }
#pragma unroll
    for (int q = 0; q < SW; q++) {
      const float k1 = frcp(fmaf(lam, pp[q], 1.f));
      P[q] = k1 * pp[q];
      m[q] = k1 * mp[q];
    }
  });
  // the chunk's last step, with d, r of step t1 (none at the sequence's end)
  float dn[SW], rn[SW];
  const bool more = g.t1 < a.e.T;
  if (more) elkc_next<CELL, ST>(a, g, w, first, s, dn, rn);
#pragma unroll
  for (int q = 0; q < SW; q++) {
    float G = 0.f, e = m[q];
    if (more) {
      const float pp = fmaf(dn[q] * dn[q], P[q], 1.f);
      G = P[q] * dn[q] * frcp(pp);
      e = fmaf(-G, fmaf(dn[q], m[q], rn[q]), m[q]);
    } else {
      dn[q] = 0.f;
      rn[q] = 0.f;
    }
    Sa[q] = fmaf(R[q], e, Sa[q]);
    R[q] *= G;
  }
  put_chunk(sub0 + (g.t1 - 1 - g.t0) / LC, dn, rn, s);
  if (!g.on) return;
#pragma unroll
  for (int q = 0; q < SW; q++) {  // into the filter maps' space, free once their carries are taken
    a.fagg[g.ch * 2 * S + col + q] = RF[q];
    a.fagg[g.ch * 2 * S + S + col + q] = SF[q];
  }
}

template <int CELL, typename ST>
__global__ __launch_bounds__(256) void k_elkc_apply(const ElkChanArgs a) {
  __shared__ int s_stop;
  __shared__ unsigned s_dmax[4];
  if (sweep_is_stopped(a.e.st, &s_stop)) return;
  constexpr int SW = elkc_sw<CELL>(), LC = elkc_len<CELL>();
  const ElkcGeom g = elkc_geom<LC>(a, a.e.cps, a.e.nch);
  const bool first = a.e.k == 1;
  const int S = a.e.S, T = a.e.T;
  unsigned dmax = 0;
  if (g.wave_on) {
    const ChanW w = elkc_weights<ST, CELL>(a, g.c);
    float s[SW], P[SW], m[SW], Gs[LC][SW], Es[LC][SW];
    // the previous chunk's last state as the smoother pass saw it (this
    // pass may already have overwritten it)
    if (g.t0 == 0) elkc_ld_h0<ST, SW>(a, g.b, g.c, s);
#pragma unroll
    for (int q = 0; q < SW; q++) {
      if (g.t0 > 0) s[q] = a.hb[(g.ch - 1) * S + (size_t)g.c * SW + q];
      const float *x = a.fsub + g.ch * 2 * S + (size_t)g.c * SW + q;
      P[q] = x[0];
      m[q] = x[S];
    }
    elkc_gains<CELL, ST, LC>(a, g, w, first, s, P, m, [&](int i, int q, float G, float e) {
#pragma unroll
      for (int ii = 0; ii < LC; ii++)  // i is a compile-time index once unrolled
        if (ii == i) {
          Gs[ii][q] = G;
          Es[ii][q] = e;
        }
    });
    // m^s entering from the right: the filter chunk's carry through the
    // later apply chunks of the same filter chunk
    float y[SW];
    const int jf = g.j / ELKC_SUB, kk0 = g.j % ELKC_SUB;
    const size_t fch = (size_t)g.b * a.cpf + jf, sub0 = (size_t)g.b * a.e.cps + (size_t)jf * ELKC_SUB;
#pragma unroll
    for (int q = 0; q < SW; q++) y[q] = a.fcar[fch * S + (size_t)g.c * SW + q];
    for (int kk = ELKC_SUB - 1; kk > kk0; kk--) {
      if (jf * ELKC_SUB + kk >= a.e.cps) continue;
#pragma unroll
      for (int q = 0; q < SW; q++) {
        const float *x = a.e.r3 + (sub0 + kk) * 2 * S + (size_t)g.c * SW + q;
        y[q] = fmaf(x[0], y[q], x[S]);
      }
    }
    ST *h = (ST *)a.e.h;
    const ElkcRows rs = elkc_rows<ST>(a, g, g.t0, g.t1 - g.t0);
#pragma unroll
    for (int i = LC - 1; i >= 0; i--) {
      if (g.t0 + i < g.t1) {
        const size_t row = (size_t)g.b * T + g.t0 + i;
        float hv[SW];
        if (first) {
#pragma unroll
          for (int q = 0; q < SW; q++) hv[q] = 0.f;
        } else {
          elkc_bld<ST, SW>(rs.H, (unsigned)(i * S + g.c * SW) * (unsigned)sizeof(ST), hv);
        }
#pragma unroll
        for (int q = 0; q < SW; q++) {
          y[q] = fmaf(Gs[i][q], y[q], Es[i][q]);
          hv[q] += y[q];
          const unsigned u = __float_as_uint(fabsf(y[q]));
          dmax = (g.on && u > dmax) ? u : dmax;
        }
        if (g.on) st_vec<ST, SW>(h + row * S + (size_t)g.c * SW, hv);
      }
    }
  }
  dmax = wave_max_u32(dmax);
  if ((threadIdx.x & 63) == 0) s_dmax[threadIdx.x >> 6] = dmax;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned mx = s_dmax[0];
    for (int q = 1; q < 4; q++) mx = s_dmax[q] > mx ? s_dmax[q] : mx;
    max_agent(&a.e.st->dslot[a.e.k & 3][blockIdx.x % PR_DSHARDS], mx);
  }
}

template <int CELL, typename ST>
static void launch_elkc(ElkChanArgs &a, hipStream_t s) {
  const int CG = (a.n + 63) / 64;
  const unsigned gchunks = (unsigned)(((size_t)a.e.nch * CG + 3) / 4);
  const unsigned gfchunks = (unsigned)(((size_t)a.nchf * CG + 3) / 4);
  const unsigned gcarry = (unsigned)(((size_t)a.e.B * a.e.S + 63) / 64);
  hipLaunchKernelGGL((k_elkc_filter<CELL, ST>), dim3(gfchunks), dim3(256), 0, s, a);
  hipLaunchKernelGGL(k_elkc_filter_carry, dim3(gcarry), dim3(64), 0, s, a);
  hipLaunchKernelGGL((k_elkc_smooth<CELL, ST>), dim3(gfchunks), dim3(256), 0, s, a);
  hipLaunchKernelGGL(k_elkc_smooth_carry, dim3(gcarry), dim3(64), 0, s, a);
  hipLaunchKernelGGL((k_elkc_apply<CELL, ST>), dim3(gchunks), dim3(256), 0, s, a);
}

hipError_t launch_elk_sweep(ElkArgs &a, hipStream_t s) {
  const int CG = (a.S + a.sp - 1) / a.sp, cpw = 64 / a.sp;
  const unsigned gchunks = (unsigned)((((size_t)a.nch + cpw - 1) / cpw * CG + 3) / 4);
  const unsigned gcarry = (unsigned)(((size_t)a.B * a.S + 3) / 4);
  hipLaunchKernelGGL(k_elk_filter, dim3(gchunks), dim3(256), 0, s, a);
  hipLaunchKernelGGL(k_elk_filter_carry, dim3(gcarry), dim3(256), 0, s, a);
  hipLaunchKernelGGL(k_elk_gains, dim3(gchunks), dim3(256), 0, s, a);
  hipLaunchKernelGGL(k_elk_smooth_carry, dim3(gcarry), dim3(256), 0, s, a);
  if (a.h_bf16) hipLaunchKernelGGL(k_elk_apply<uint16_t>, dim3(gchunks), dim3(256), 0, s, a);
  else hipLaunchKernelGGL(k_elk_apply<float>, dim3(gchunks), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_elk_chan_sweep(int cell, bool bf16, ElkChanArgs &a, hipStream_t s) {
  if (cell == C_GRU_DIAG) {
    if (bf16) launch_elkc<C_GRU_DIAG, uint16_t>(a, s);
    else launch_elkc<C_GRU_DIAG, float>(a, s);
  } else {
    constexpr int C = C_LSTM + 16 * APX_DIAG;
    if (bf16) launch_elkc<C, uint16_t>(a, s);
    else launch_elkc<C, float>(a, s);
  }
  return hipGetLastError();
}

}  // namespace pr

// Channel-parallel building blocks for per-channel state (diagonal ParaGRU,
// SW = 1; CIFG/peephole ParaLSTM with a 2x2 block Jacobian, SW = 2): buffer
// loads, per-channel weights, the start-of-sweep stop check, the standalone
// diagonal / 2x2-block affine scan, and the fixed-order reduction of the
// adjoint's weight partials.  The Newton sweep and the adjoint are streaming
// passes (k_chan2.hip).
//
// Channels are independent, so a scan runs per (sequence, channel) along time
// (Para-Seq README, Main features: diagonal and 2x2 block scans).  Layout of
// the standalone scan: a lane owns CPL adjacent channels (coalesced loads
// across the wavefront), a tile is 4 wavefronts x TW steps of those 64*CPL
// channels; each lane composes its TW steps serially per channel, the 4
// wavefronts combine in LDS, and consecutive time tiles of a stripe (sequence
// b, channel group) chain through a decoupled look-back whose descriptors are
// per channel.  A persistent grid walks the tiles in increasing time-major
// order.
#pragma once

#include "cells_chan.h"
#include "internal.h"
#include "pipe.h"  // buffer-resource loads and stores

namespace pr {

// Packed buffer loads: BYTES (2, 4, 8 or 16) into 32-bit words as stored (a
// 2-byte value in the low half); out-of-range offsets read zero.  A tile's
// loads are issued together, unconditionally, so they are all in flight
// before the first one is waited for.
template <int BYTES>
__device__ inline void bldw(Rsrc r, unsigned off, unsigned *w) {
  if constexpr (BYTES == 2) {
    w[0] = ld_u16(r, off);
  } else if constexpr (BYTES == 4) {
    w[0] = ld_u32(r, off);
  } else if constexpr (BYTES == 8) {
    const u32x2 u = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    w[0] = u.x; w[1] = u.y;
  } else {
    static_assert(BYTES == 16, "unsupported access width");
    const u32x4 u = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    w[0] = u.x; w[1] = u.y; w[2] = u.z; w[3] = u.w;
  }
}
// value i of packed words w (storage type ST)
template <typename ST>
__device__ inline float unpackw(const unsigned *w, int i) {
  if constexpr (sizeof(ST) == 2) return __uint_as_float((i & 1) ? (w[i >> 1] & 0xffff0000u) : (w[i >> 1] << 16));
  else return __uint_as_float(w[i]);
}
template <typename ST, int CNT>
constexpr int words_of() {
  return (CNT * (int)sizeof(ST) + 3) / 4;
}

template <typename ST, int CNT>
__device__ inline void ld_vec(const ST *p, float *out) {
  if constexpr (sizeof(ST) * CNT == 16) {
    uint4 u = *reinterpret_cast<const uint4 *>(p);
    unsigned w[4] = {u.x, u.y, u.z, u.w};
    if constexpr (sizeof(ST) == 4) {
#pragma unroll
      for (int i = 0; i < 4; i++) out[i] = __uint_as_float(w[i]);
    } else {
#pragma unroll
      for (int i = 0; i < 8; i++) out[i] = __uint_as_float((w[i / 2] >> (16 * (i & 1))) << 16);
    }
  } else if constexpr (sizeof(ST) * CNT == 8) {
    uint2 u = *reinterpret_cast<const uint2 *>(p);
    unsigned w[2] = {u.x, u.y};
    if constexpr (sizeof(ST) == 4) {
      out[0] = __uint_as_float(w[0]);
      out[1] = __uint_as_float(w[1]);
    } else {
#pragma unroll
      for (int i = 0; i < 4; i++) out[i] = __uint_as_float((w[i / 2] >> (16 * (i & 1))) << 16);
    }
  } else if constexpr (sizeof(ST) * CNT == 4) {
    unsigned u = *reinterpret_cast<const unsigned *>(p);
    if constexpr (sizeof(ST) == 4) {
      out[0] = __uint_as_float(u);
    } else {
      out[0] = __uint_as_float(u << 16);
      out[1] = __uint_as_float(u & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < CNT; i++) out[i] = ldf(p, i);
  }
}

template <typename ST, int CNT>
__device__ inline void st_vec(ST *p, const float *in) {
  if constexpr (sizeof(ST) == 2 && CNT % 2 == 0) {
    unsigned w[CNT / 2];
#pragma unroll
    for (int i = 0; i < CNT / 2; i++) w[i] = (unsigned)f2bf(in[2 * i]) | ((unsigned)f2bf(in[2 * i + 1]) << 16);
    if constexpr (CNT == 2) *reinterpret_cast<unsigned *>(p) = w[0];
    else if constexpr (CNT == 4) *reinterpret_cast<uint2 *>(p) = make_uint2(w[0], w[1]);
    else {
#pragma unroll
      for (int i = 0; i < CNT / 2; i++) reinterpret_cast<unsigned *>(p)[i] = w[i];
    }
  } else if constexpr (sizeof(ST) == 4 && CNT == 2) {
    *reinterpret_cast<float2 *>(p) = make_float2(in[0], in[1]);
  } else if constexpr (sizeof(ST) == 4 && CNT == 4) {
    *reinterpret_cast<float4 *>(p) = make_float4(in[0], in[1], in[2], in[3]);
  } else {
#pragma unroll
    for (int i = 0; i < CNT; i++) stf(p, i, in[i]);
  }
}

// Tile geometry and stripe bookkeeping shared by the kernels.
template <int SW, int CPL, int TW>
struct ChanGeom {
  static constexpr int CH = 64 * CPL;   // channels per tile
  static constexpr int TT = 4 * TW;     // steps per tile
  static constexpr int AW = SW * SW + SW;
};

// Combine the four wavefronts' per-channel aggregates (wave w covers steps
// [w*TW, (w+1)*TW) of the tile).  pre[c] = composition of the waves before
// this one, tot[c] = tile aggregate.  Contains one __syncthreads.
template <int SW, int CPL>
__device__ inline void chan_combine(const Op<SW> (&agg)[CPL], Op<SW> (&pre)[CPL], Op<SW> (&tot)[CPL],
                                    float *s_agg /*[4][64*CPL][SW*SW+SW]*/) {
  constexpr int AW = SW * SW + SW, CH = 64 * CPL;
  const int lane = threadIdx.x & 63, wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
  for (int c = 0; c < CPL; c++) {
    float *d = s_agg + ((size_t)wid * CH + lane * CPL + c) * AW;
#pragma unroll
    for (int i = 0; i < SW * SW; i++) d[i] = agg[c].A[i];
#pragma unroll
    for (int i = 0; i < SW; i++) d[SW * SW + i] = agg[c].b[i];
  }
  __syncthreads();
#pragma unroll
  for (int c = 0; c < CPL; c++) {
    Op<SW> p = op_identity<SW>(), t = op_identity<SW>();
#pragma unroll
    for (int w = 0; w < 4; w++) {
      const float *s = s_agg + ((size_t)w * CH + lane * CPL + c) * AW;
      Op<SW> o;
#pragma unroll
      for (int i = 0; i < SW * SW; i++) o.A[i] = s[i];
#pragma unroll
      for (int i = 0; i < SW; i++) o.b[i] = s[SW * SW + i];
      if (w < wid) p = compose(o, p);
      t = compose(o, t);
    }
    pre[c] = p;
    tot[c] = t;
  }
}

// Per-lane decoupled look-back over the time tiles of one stripe (run by
// wavefront 0; lane l owns the same CPL channels in every tile of the
// stripe).  Descriptor words: agg [tile][64*CPL][SW*SW+SW], incl
// [tile][64*CPL][SW], each tagged with the sweep number.  Each round trip
// reads W predecessors; carry[c] receives the state after tile j - 1.
template <int SW, int CPL, int W>
__device__ inline void chan_lookback(const Op<SW> (&tot)[CPL], int j, int k, bool active,
                                     unsigned long long *agg, unsigned long long *incl, float (&carry)[CPL][SW],
                                     SolveState *st) {
  constexpr int AW = SW * SW + SW, CH = 64 * CPL;
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int c = 0; c < CPL; c++)
#pragma unroll
    for (int i = 0; i < SW; i++) carry[c][i] = 0.f;
  if (!active) return;
  if (j > 0) {
#pragma unroll
    for (int c = 0; c < CPL; c++) {
      unsigned long long *d = agg + ((size_t)j * CH + lane * CPL + c) * AW;
#pragma unroll
      for (int i = 0; i < SW * SW; i++) desc_put(d + i, tag_agg(k), tot[c].A[i]);
#pragma unroll
      for (int i = 0; i < SW; i++) desc_put(d + SW * SW + i, tag_agg(k), tot[c].b[i]);
    }
    Op<SW> acc[CPL];
#pragma unroll
    for (int c = 0; c < CPL; c++) acc[c] = op_identity<SW>();
    int p0 = j - 1, spins = 0;
    bool done = false;
    while (!done) {
      unsigned long long wi[W][CPL][SW], wa[W][CPL][AW];
#pragma unroll
      for (int q = 0; q < W; q++) {
        const int p = p0 - q;
#pragma unroll
        for (int c = 0; c < CPL; c++) {
#pragma unroll
          for (int i = 0; i < SW; i++)
            wi[q][c][i] = p >= 0 ? ld_agent64(incl + ((size_t)p * CH + lane * CPL + c) * SW + i) : 0ull;
#pragma unroll
          for (int i = 0; i < AW; i++)
            wa[q][c][i] = p >= 0 ? ld_agent64(agg + ((size_t)p * CH + lane * CPL + c) * AW + i) : 0ull;
        }
      }
      int q = 0;
      for (; q < W; q++) {
        bool hi = true, ha = true;
#pragma unroll
        for (int c = 0; c < CPL; c++) {
#pragma unroll
          for (int i = 0; i < SW; i++) hi = hi && (unsigned)(wi[q][c][i] >> 32) == tag_incl(k);
#pragma unroll
          for (int i = 0; i < AW; i++) ha = ha && (unsigned)(wa[q][c][i] >> 32) == tag_agg(k);
        }
        if (hi) {
#pragma unroll
          for (int c = 0; c < CPL; c++) {
            float v[SW];
#pragma unroll
            for (int i = 0; i < SW; i++) v[i] = __uint_as_float((unsigned)wi[q][c][i]);
            op_apply(acc[c], v, carry[c]);
          }
          done = true;
          break;
        }
        if (!ha) break;  // predecessor not published yet: retry from here
#pragma unroll
        for (int c = 0; c < CPL; c++) {
          Op<SW> o;
#pragma unroll
          for (int i = 0; i < SW * SW; i++) o.A[i] = __uint_as_float((unsigned)wa[q][c][i]);
#pragma unroll
          for (int i = 0; i < SW; i++) o.b[i] = __uint_as_float((unsigned)wa[q][c][SW * SW + i]);
          acc[c] = compose(acc[c], o);
        }
      }
      if (!done) {
        if (q < W) {
          if (++spins > PR_SPIN_LIMIT) {  // reported by the host; a NaN carry poisons the rest
            spin_fault(st);
#pragma unroll
            for (int c = 0; c < CPL; c++)
#pragma unroll
              for (int i = 0; i < SW; i++) carry[c][i] = __builtin_nanf("");
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
        p0 -= q;
      }
    }
  }
#pragma unroll
  for (int c = 0; c < CPL; c++) {
    float inc[SW];
    op_apply(tot[c], carry[c], inc);
    unsigned long long *d = incl + ((size_t)j * CH + lane * CPL + c) * SW;
#pragma unroll
    for (int i = 0; i < SW; i++) desc_put(d + i, tag_incl(k), inc[i]);
  }
}

template <typename ST, int CELL>
__device__ inline ChanW load_chan_w(const ChanArgs &a, int c) {
  const ST *Wh = (const ST *)a.Wh, *bh = (const ST *)a.bh, *pp = (const ST *)a.peep;
  const int n = a.n;
  // all eight loads unconditional (an absent vector reads W_h instead and is
  // replaced by zeros), so they are in flight together
  const ST *bq = bh ? bh : Wh, *pq = pp ? pp : Wh;
  ChanW w;
  w.a0 = ldf(Wh, c);
  w.a1 = ldf(Wh, (size_t)n + c);
  w.a2 = ldf(Wh, (size_t)2 * n + c);
  const float b0 = ldf(bq, c), b1 = ldf(bq, (size_t)n + c), b2 = ldf(bq, (size_t)2 * n + c);
  const float p0 = ldf(pq, c), p1 = ldf(pq, (size_t)n + c);
  w.b0 = bh ? b0 : 0.f;
  w.b1 = bh ? b1 : 0.f;
  w.b2 = bh ? b2 : 0.f;
  w.p0 = pp ? p0 : 0.f;
  w.p1 = pp ? p1 : 0.f;
  chan_w_scale<CELL>(w);
  return w;
}

// Stop rule on the previous sweep's measure; block 0 finalises the history
// and clears the next sweep's shards.  Returns true when the solve stopped.
__device__ inline bool chan_stopped(const ChanArgs &a, int *s_stop) {
  const int k = a.k;
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int stop = ld_agent(&a.st->stopped) != 0;
    if (!stop && k >= 2) {
      unsigned d = wave_max_u32(ld_agent(&a.st->dslot[(k - 1) & 3][lane]));
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

// ---------------------------------------------------------------------------
// standalone scan with given operators (fp32):  y_t = A_t y_{t-1} + b_t, or
// in reverse time y_t = A_t y_{t+1} + b_t.  SW = 1: A, b [B,T,n];
// SW = 2: A [B,T,n,2,2], b [B,T,n,2].
// ---------------------------------------------------------------------------
template <int SW, int CPL, int TW>
__global__ __launch_bounds__(256) void k_chan_scan(const ChanArgs a) {
  using Gm = ChanGeom<SW, CPL, TW>;
  constexpr int CH = Gm::CH, TT = Gm::TT, AW = Gm::AW;
  __shared__ float s_agg[4 * CH * AW];
  __shared__ float s_carry[CH * SW];
  const int tid = threadIdx.x, lane = tid & 63, wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int T = a.T, n = a.n, S = SW * n;
  const int CG = (n + CH - 1) / CH;
  for (int id = blockIdx.x; id < a.ntiles; id += gridDim.x) {
    const int j = id / a.stripes, stripe = id % a.stripes;
    const int b = stripe / CG, cg = stripe % CG;
    const int c0 = cg * CH + lane * CPL;
    const bool active = c0 < n;
    const int s0 = j * TT + wid * TW;  // scan positions of this wave
    Op<SW> el[TW][CPL], agg[CPL];
#pragma unroll
    for (int c = 0; c < CPL; c++) agg[c] = op_identity<SW>();
#pragma unroll
    for (int s = 0; s < TW; s++) {
      const int sp = s0 + s;
      const int t = a.reverse ? T - 1 - sp : sp;
#pragma unroll
      for (int c = 0; c < CPL; c++) {
        el[s][c] = op_identity<SW>();
        if (active && sp < T) {
          const size_t e = ((size_t)b * T + t) * n + c0 + c;
#pragma unroll
          for (int i = 0; i < SW * SW; i++) el[s][c].A[i] = a.A[e * SW * SW + i];
#pragma unroll
          for (int i = 0; i < SW; i++) el[s][c].b[i] = a.b[e * SW + i];
          agg[c] = compose(el[s][c], agg[c]);
        }
      }
    }
    Op<SW> pre[CPL], tot[CPL];
    chan_combine<SW, CPL>(agg, pre, tot, s_agg);
    if (wid == 0) {
      float carry[CPL][SW];
      chan_lookback<SW, CPL, 4>(tot, j, 1, active, a.agg + (size_t)stripe * a.tps * CH * AW,
                                a.incl + (size_t)stripe * a.tps * CH * SW, carry, a.st);
#pragma unroll
      for (int c = 0; c < CPL; c++)
#pragma unroll
        for (int i = 0; i < SW; i++) s_carry[(lane * CPL + c) * SW + i] = carry[c][i];
    }
    __syncthreads();
    float y[CPL][SW];
#pragma unroll
    for (int c = 0; c < CPL; c++) op_apply(pre[c], &s_carry[(lane * CPL + c) * SW], y[c]);
#pragma unroll
    for (int s = 0; s < TW; s++) {
      const int sp = s0 + s;
      if (active && sp < T) {
        const int t = a.reverse ? T - 1 - sp : sp;
#pragma unroll
        for (int c = 0; c < CPL; c++) {
          float ny[SW];
          op_apply(el[s][c], y[c], ny);
#pragma unroll
          for (int i = 0; i < SW; i++) {
            y[c][i] = ny[i];
            a.y[(((size_t)b * T + t) * n + c0 + c) * SW + i] = ny[i];
          }
        }
      }
    }
    __syncthreads();
  }
}

}  // namespace pr

namespace pr {

// ---------------------------------------------------------------------------
// adjoint weight-gradient partials per channel:
// [a0 a1 a2 | b0 b1 b2 | p0 p1 | sum dU0 dU1 dU2] (CHAN_P values)
// ---------------------------------------------------------------------------
constexpr int CHAN_P = 11;

// Per-tile partials [stripe][tile][CH][CHAN_P] summed in two fixed-order
// stages: split q of the (sequence, tile) terms of every (channel, slot) into
// red[q][n][CHAN_P] (fp64), then the splits in order into the gradients.
template <int CH>
__global__ __launch_bounds__(256) void k_chan_red_split(const ChanArgs a, double *red) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  const int n = a.n;
  if (e >= n * CHAN_P) return;
  const int c = e / CHAN_P, p = e % CHAN_P;
  const int CG = (n + CH - 1) / CH, cg = c / CH, cl = c % CH;
  const int terms = (a.stripes / CG) * a.tps, per = (terms + gridDim.y - 1) / gridDim.y;
  const int q0 = blockIdx.y * per, q1 = min(terms, q0 + per);
  double s = 0.0;
#pragma unroll 8
  for (int q = q0; q < q1; q++) {
    const int stripe = (q / a.tps) * CG + cg, j = q % a.tps;
    s += (double)a.part[(((size_t)stripe * a.tps + j) * CH + cl) * CHAN_P + p];
  }
  red[(size_t)blockIdx.y * n * CHAN_P + e] = s;
}

template <int SPLITS>
__global__ __launch_bounds__(256) void k_chan_red_final(const ChanArgs a, const double *red, float *dWh,
                                                        float *dbh, float *dpeep, float *dbx) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  const int n = a.n;
  if (e >= n * CHAN_P) return;
  const int c = e / CHAN_P, p = e % CHAN_P;
  double s = 0.0;
  for (int q = 0; q < SPLITS; q++) s += red[(size_t)q * n * CHAN_P + e];
  const float v = (float)s;
  if (p < 3) { if (dWh) dWh[(size_t)p * n + c] = v; }
  else if (p < 6) { if (dbh) dbh[(size_t)(p - 3) * n + c] = v; }
  else if (p < 8) { if (dpeep && a.SW == 2) dpeep[(size_t)(p - 6) * n + c] = v; }
  else { if (dbx) dbx[(size_t)(p - 8) * n + c] = v; }
}

}  // namespace pr

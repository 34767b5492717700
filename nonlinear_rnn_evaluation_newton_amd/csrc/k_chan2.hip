// Newton sweep of the per-channel cells (diagonal ParaGRU; CIFG/peephole
// ParaLSTM with 2x2 blocks) as streaming passes with no chain between tiles.
//
// The sweep's linear recurrence dh_t = J_t dh_{t-1} + r_t (DEER summary,
// Approach; Para-Seq README, Main features: diagonal and 2x2 block scans) is
// solved tile by tile from per-tile carries, and the carries come from the
// tiles' aggregates by a short scan.  The aggregates of sweep k + 1 depend
// only on the iterate that sweep k writes, so the pass that applies sweep k
// also composes them, step by step, right after it has written each new
// state.  Per sweep:
//
//   k_chan_carry   the first step of every tile (whose linearisation point is
//                  the previous tile's last state) is evaluated and composed
//                  with the tile's partial aggregate; an exclusive scan over
//                  each stripe's tiles gives the carries (dh entering a tile);
//   k_chan_pass    each wavefront walks one tile (64 steps x 64*CPL channels)
//                  serially: applies sweep k from its carry (cell, Jacobian,
//                  residual, dh, h += dh, stores, max |dh|) and composes the
//                  partial aggregate of sweep k + 1 at the new iterate.
//
// Before sweep 1 a pass composes the aggregates at the initial guess only.
// When the sweep count is fixed and an adjoint follows, the last pass
// composes the adjoint's tile aggregates instead (ADJ): the elements
// (J_t^T, J_t^T g_t) at the final iterate, with the cell's own Jacobian,
// which the adjoint would otherwise evaluate in a pass of its own.
// The iterate is read once and written once per sweep, like a single-pass
// scan, at the price of a second cell evaluation per step; no wavefront ever
// waits for another, so there is no look-back latency and no co-residency
// requirement.  Both sides of a tile boundary use the stored (rounded) state
// of the previous tile's last step, so aggregates and updates agree exactly.
//
// The sweep kernels' cell argument may carry a Jacobian approximation
// (cell_apx: the 2x2 blocks' diagonal, or zero for Jacobi sweeps); it changes
// the operator of the linear recurrence and nothing else.
#include <type_traits>

#include "k_chan_impl.h"

namespace pr {

constexpr int C2_P = 4;                 // steps per load group (two groups in flight)
constexpr int C2_NG = CHAN2_TT / C2_P;  // load groups per tile
constexpr int C2_CW = 16;               // wavefronts per carry block
constexpr int C2_R = 4;                 // tiles per carry chunk (their loads are issued together)

// Store CNT values as ST (bf16: round to nearest even) with cache policy POL
// (SC_NT for outputs nothing in the call reads back); out-of-range offsets
// are dropped.
template <typename ST, int CNT, int POL = 0>
__device__ inline void bst(Rsrc r, unsigned off, const float *in) {
  constexpr int BYTES = CNT * (int)sizeof(ST);
  auto word = [&](int i) -> unsigned {
    if constexpr (sizeof(ST) == 2) return (unsigned)f2bf(in[2 * i]) | ((unsigned)f2bf(in[2 * i + 1]) << 16);
    else return __float_as_uint(in[i]);
  };
  if constexpr (BYTES == 2) {
    __builtin_amdgcn_raw_buffer_store_b16(f2bf(in[0]), r, off, 0, POL);
  } else if constexpr (BYTES == 4) {
    __builtin_amdgcn_raw_buffer_store_b32(word(0), r, off, 0, POL);
  } else if constexpr (BYTES == 8) {
    u32x2 v;
    v.x = word(0); v.y = word(1);
    __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, POL);
  } else {
    static_assert(BYTES == 16, "unsupported access width");
    u32x4 v;
    v.x = word(0); v.y = word(1); v.z = word(2); v.w = word(3);
    __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, POL);
  }
}

// Store CNT values that are already exact in ST (bf16 values rounded by
// as_stored): a bf16 pair packs with one byte permute of the two high halves.
template <typename ST, int CNT>
__device__ inline void bst_exact(Rsrc r, unsigned off, const float *in) {
  if constexpr (sizeof(ST) == 2 && CNT == 2) {
    st_u32(r, off, __builtin_amdgcn_perm(__float_as_uint(in[1]), __float_as_uint(in[0]), 0x07060302u));
  } else {
    bst<ST, CNT>(r, off, in);
  }
}

// the value a float takes once stored as ST
template <typename ST>
__device__ inline float as_stored(float v) {
  if constexpr (sizeof(ST) == 2) return bf2f(f2bf(v));
  else return v;
}

// State before step t0 of tile L at iterate k - 1 (fp32, as stored; CPL
// channels of SW values): h0 for the first tile, the previous tile's last
// state kept by pass k - 1, or the initial guess 0.
template <typename ST, int CPL, int SW, int CH>
__device__ inline void state_before(const ChanArgs &a, int k, int t0, int b, int L, int c0, int lane, bool active,
                                    float *s) {
  // both candidate loads are issued unconditionally (from valid addresses),
  // then one is selected
  const bool from_h0 = t0 == 0 && a.h0 != nullptr, from_bnd = t0 > 0 && k >= 2;
  const float *bp =
      a.bnd + ((size_t)((k - 1) & 1) * a.ntiles + (from_bnd ? L - 1 : 0)) * CH * SW + (size_t)lane * CPL * SW;
  const ST *hp = from_h0 ? (const ST *)a.h0 + (size_t)b * SW * a.n + (size_t)(active ? c0 : 0) * SW : (const ST *)a.Wh;
#pragma unroll
  for (int i = 0; i < CPL * SW; i++) {
    const float vb = bp[i], vh = ldf(hp, i);
    s[i] = !active ? 0.f : from_bnd ? vb : from_h0 ? vh : 0.f;
  }
}

template <int CELL, typename ST, int CPL, bool APPLY, bool NEXT, bool ADJ = false>
__global__ __launch_bounds__(256) void k_chan_pass(const ChanArgs a) {
  static_assert(!ADJ || (APPLY && !NEXT), "the adjoint's aggregates come with the last applying pass");
  constexpr int SW = cell_code(CELL) == C_LSTM ? 2 : 1, CH = 64 * CPL, AW = SW * SW + SW, ES = (int)sizeof(ST);
  constexpr int UW = words_of<ST, CPL>(), HW = words_of<ST, CPL * SW>(), TT = CHAN2_TT;
  __shared__ int s_stop;
  __shared__ unsigned s_dmax[4];
  const int k = a.k;
  if (APPLY && chan_stopped(a, &s_stop)) return;
  const int lane = threadIdx.x & 63, wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tile = blockIdx.x * 4 + wid;
  const int T = a.T, n = a.n, S = SW * n;
  unsigned dmax = 0;
  if (tile < a.ntiles) {
    const int j = tile / a.stripes, stripe = tile % a.stripes;
    const int CG = (n + CH - 1) / CH, b = stripe / CG;
    const int c0 = (stripe % CG) * CH + lane * CPL;
    const bool active = c0 < n;  // n is a multiple of CPL
    const int L = stripe * a.tps + j, t0 = j * TT, nrows = min(TT, T - t0);
    ChanW w[CPL];
#pragma unroll
    for (int c = 0; c < CPL; c++) w[c] = load_chan_w<ST, CELL>(a, active ? c0 + c : 0);

    // the tile's rows; the iterate is read from sweep 2 on (sweep 1 starts from 0)
    const size_t row0 = (size_t)b * T + t0;
    const Rsrc ru = sc_rsrc((const ST *)a.U + row0 * 3 * n, (unsigned)(nrows * 3 * n * ES));
    const Rsrc rh = sc_rsrc((APPLY && k >= 2) ? (const ST *)a.h + row0 * S : nullptr, (unsigned)(nrows * S * ES));
    const Rsrc rw = sc_rsrc((ST *)a.h + row0 * S, (unsigned)(nrows * S * ES));
    const Rsrc rg = sc_rsrc(ADJ ? (const ST *)a.g + row0 * S : nullptr, (unsigned)(nrows * S * ES));

    float s_old[CPL * SW], s_new[CPL * SW], dh[CPL * SW];
    Op<SW> agg[CPL];
#pragma unroll
    for (int c = 0; c < CPL; c++) agg[c] = op_identity<SW>();
    state_before<ST, CPL, SW, CH>(a, APPLY ? k : 1, t0, b, L, c0, lane, active, s_old);
#pragma unroll
    for (int i = 0; i < CPL * SW; i++) {
      s_new[i] = s_old[i];
      dh[i] = 0.f;
    }
    if constexpr (APPLY) {
      const float *cp = (const float *)a.incl + ((size_t)L * CH + lane * CPL) * SW;
#pragma unroll
      for (int i = 0; i < CPL * SW; i++) dh[i] = cp[i];
    }

    // Offsets carry bit 31 for idle lanes (outside every resource); rows past
    // the tile or past T lie outside the tile's resources.  No selects or
    // branches sit between the loads, so they all stay in flight.
    // The lane parts of the offsets (with the idle bit) are formed once; each
    // access adds its row's wave-uniform part (one add; the sum stays below
    // 2^32 and keeps bit 31).
    const unsigned lane_oob = active ? 0u : SC_OOB;
    const unsigned ulane = (unsigned)(c0 * ES) | lane_oob, hlane = (unsigned)(c0 * SW * ES) | lane_oob;
    unsigned ua[C2_P][3][UW], ha[C2_P][HW], ub[C2_P][3][UW], hb[C2_P][HW];
    unsigned ga[ADJ ? C2_P : 1][HW], gb[ADJ ? C2_P : 1][HW];  // ADJ: the upstream gradient g
    auto load = [&](int g, unsigned (&u)[C2_P][3][UW], unsigned (&h)[C2_P][HW],
                    unsigned (&gr)[ADJ ? C2_P : 1][HW]) __attribute__((always_inline)) {
#pragma unroll
      for (int q = 0; q < C2_P; q++) {
        const int s = g * C2_P + q;
#pragma unroll
        for (int gi = 0; gi < 3; gi++) bldw<CPL * ES>(ru, ulane + (unsigned)((s * 3 * n + gi * n) * ES), u[q][gi]);
        bldw<CPL * SW * ES>(rh, hlane + (unsigned)(s * S * ES), h[q]);
        if constexpr (ADJ) bldw<CPL * SW * ES>(rg, hlane + (unsigned)(s * S * ES), gr[q]);
      }
    };
    // FULL: every lane active and every step inside [0, T) (all tiles but a
    // sequence's last one when n fills the stripe): no identity selects
    auto steps = [&](auto full, int g, const unsigned (&u)[C2_P][3][UW], const unsigned (&h)[C2_P][HW],
                     const unsigned (&gr)[ADJ ? C2_P : 1][HW]) __attribute__((always_inline)) {
      constexpr bool FULL = decltype(full)::value;
#pragma unroll
      for (int q = 0; q < C2_P; q++) {
        const int s = g * C2_P + q;
        const bool valid = FULL || (active && s < nrows);
        float hn[CPL * SW];
#pragma unroll
        for (int c = 0; c < CPL; c++) {
          const float uc[3] = {unpackw<ST>(u[q][0], c), unpackw<ST>(u[q][1], c), unpackw<ST>(u[q][2], c)};
          float hold[SW];
#pragma unroll
          for (int i = 0; i < SW; i++) hold[i] = unpackw<ST>(h[q], c * SW + i);
          if constexpr (APPLY) {
            // sweep k at this step: J, r at the old iterate, then the update
            float f[SW], J[SW * SW], nd[SW];
            chan_cell<CELL>(&s_old[c * SW], uc, w[c], f, J);
#pragma unroll
            for (int i = 0; i < SW; i++) {
              float v = f[i] - hold[i];
#pragma unroll
              for (int m = 0; m < SW; m++) v = fmaf(J[i * SW + m], dh[c * SW + m], v);
              nd[i] = v;
            }
#pragma unroll
            for (int i = 0; i < SW; i++) {
              dh[c * SW + i] = nd[i];
              hn[c * SW + i] = as_stored<ST>(hold[i] + nd[i]);
              const unsigned ab = valid ? __float_as_uint(nd[i]) & 0x7fffffffu : 0u;
              dmax = ab > dmax ? ab : dmax;
              s_old[c * SW + i] = hold[i];
            }
          } else {
#pragma unroll
            for (int i = 0; i < SW; i++) hn[c * SW + i] = hold[i];
          }
          if constexpr (NEXT) {
            // sweep k + 1 at this step (the tile's first step is composed by
            // the carry kernel): J, r at the new iterate
            if (s > 0) {
              float f[SW], J[SW * SW];
              chan_cell<CELL>(&s_new[c * SW], uc, w[c], f, J);
              Op<SW> e;
#pragma unroll
              for (int i = 0; i < SW; i++) e.b[i] = valid ? f[i] - hn[c * SW + i] : 0.f;
#pragma unroll
              for (int i = 0; i < SW * SW; i++) e.A[i] = valid ? J[i] : ((i % (SW + 1)) == 0 ? 1.f : 0.f);
              agg[c] = compose(e, agg[c]);
            }
          }
          if constexpr (ADJ) {
            // the adjoint's element of this step at the new iterate, with the
            // cell's own Jacobian: mu_{t-1} = J_t^T mu_t + J_t^T g_t, composed
            // so that later steps act first (the tile's first step is the
            // adjoint carry kernel's)
            if (s > 0) {
              float f[SW], J[SW * SW];
              chan_cell<cell_code(CELL)>(&s_new[c * SW], uc, w[c], f, J);
              Op<SW> e;
#pragma unroll
              for (int r = 0; r < SW; r++) {
                float v = 0.f;
#pragma unroll
                for (int q2 = 0; q2 < SW; q2++) {
                  e.A[r * SW + q2] = valid ? J[q2 * SW + r] : (r == q2 ? 1.f : 0.f);
                  v = fmaf(J[q2 * SW + r], unpackw<ST>(gr[q], c * SW + q2), v);
                }
                e.b[r] = valid ? v : 0.f;
              }
              agg[c] = compose(agg[c], e);
            }
          }
#pragma unroll
          for (int i = 0; i < SW; i++) s_new[c * SW + i] = hn[c * SW + i];
        }
        if constexpr (APPLY) bst_exact<ST, CPL * SW>(rw, hlane + (unsigned)(s * S * ES), hn);
      }
    };
    auto walk = [&](auto full) __attribute__((always_inline)) {
      load(0, ua, ha, ga);
      for (int g = 0; g < C2_NG; g += 2) {
        load(g + 1, ub, hb, gb);
        steps(full, g, ua, ha, ga);
        load(g + 2, ua, ha, ga);
        steps(full, g + 1, ub, hb, gb);
      }
    };
    const int last_c = (stripe % CG) * CH + 63 * CPL;  // first channel of lane 63
    if (nrows == TT && last_c < n) walk(std::true_type{});
    else walk(std::false_type{});
    if (active) {
      if constexpr (APPLY) {  // the tile's last state, as stored, for the next sweep's neighbour
        if (nrows == TT) {
          float *bp = a.bnd + ((size_t)(k & 1) * a.ntiles + L) * CH * SW + (size_t)lane * CPL * SW;
#pragma unroll
          for (int i = 0; i < CPL * SW; i++) bp[i] = s_new[i];
        }
      }
      if constexpr (NEXT || ADJ) {
        float *pa = (float *)a.agg + ((size_t)L * CH + lane * CPL) * AW;
#pragma unroll
        for (int c = 0; c < CPL; c++) {
#pragma unroll
          for (int i = 0; i < SW * SW; i++) pa[c * AW + i] = agg[c].A[i];
#pragma unroll
          for (int i = 0; i < SW; i++) pa[c * AW + SW * SW + i] = agg[c].b[i];
        }
      }
    }
  }
  if constexpr (APPLY) {
    dmax = wave_max_u32(dmax);
    if (lane == 0) s_dmax[wid] = dmax;
    __syncthreads();
    if (threadIdx.x == 0) {
      unsigned m = s_dmax[0];
      for (int q = 1; q < 4; q++) m = s_dmax[q] > m ? s_dmax[q] : m;
      max_agent(&a.st->dslot[k & 3][blockIdx.x % PR_DSHARDS], m);
    }
  }
}

// Carries of sweep k for one stripe (block), C2_CW wavefronts splitting its
// tiles into contiguous ranges: the first-step element of each tile composed
// under the tile's partial aggregate (written back as the full aggregate),
// the range totals combined in LDS, then the exclusive prefix walked again.
template <int CELL, typename ST, int CPL>
__global__ __launch_bounds__(64 * C2_CW) void k_chan_carry(const ChanArgs a) {
  constexpr int SW = cell_code(CELL) == C_LSTM ? 2 : 1, CH = 64 * CPL, AW = SW * SW + SW, TT = CHAN2_TT;
  constexpr int R = C2_R;
  __shared__ float s_tot[C2_CW][CH][AW];
  __shared__ int s_skip;
  const int k = a.k, lane = threadIdx.x & 63, wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // nothing to do once the previous sweep met the stop rule (its pass then
  // records the stop)
  if (threadIdx.x < 64) {  // one shard of the previous sweep's measure per lane
    int skip = ld_agent(&a.st->stopped) != 0;
    if (!skip && k >= 2) {
      const unsigned d = wave_max_u32(ld_agent(&a.st->dslot[(k - 1) & 3][threadIdx.x]));
      int status;
      skip = stop_rule(__uint_as_float(d), k - 1, a.tol, a.T, a.max_iters, &status) ? 1 : 0;
    }
    if (threadIdx.x == 0) s_skip = skip;
  }
  __syncthreads();
  if (s_skip) return;
  const int T = a.T, n = a.n, S = SW * n, stripe = blockIdx.x;
  const int CG = (n + CH - 1) / CH, b = stripe / CG;
  const int c0 = (stripe % CG) * CH + lane * CPL;
  const bool active = c0 < n;
  const int nt = a.tps, per = (nt + C2_CW - 1) / C2_CW;
  const int j0 = min(nt, wid * per), j1 = min(nt, j0 + per);
  ChanW w[CPL];
#pragma unroll
  for (int c = 0; c < CPL; c++) w[c] = load_chan_w<ST, CELL>(a, active ? c0 + c : 0);
  const ST *U = (const ST *)a.U, *H = (const ST *)a.h;
  float *pagg = (float *)a.agg;
  float *carry = (float *)a.incl;

  Op<SW> tot[CPL];
#pragma unroll
  for (int c = 0; c < CPL; c++) tot[c] = op_identity<SW>();
  for (int jc = j0; jc < j1; jc += R) {
    // every load of the chunk is issued unconditionally (idle slots read a
    // valid tile's data and are discarded), then used
    float u[R][CPL][3], hc[R][CPL * SW], sb[R][CPL * SW], pg[R][CPL][AW];
#pragma unroll
    for (int r = 0; r < R; r++) {
      const int jj = jc + r < j1 ? jc + r : j0, L = stripe * nt + jj, t0 = jj * TT;
      const int cc = active ? c0 : 0;
      const size_t row = (size_t)b * T + t0;
#pragma unroll
      for (int c = 0; c < CPL; c++)
#pragma unroll
        for (int gi = 0; gi < 3; gi++) u[r][c][gi] = ldf(U, row * 3 * n + (size_t)gi * n + cc + c);
      state_before<ST, CPL, SW, CH>(a, k, t0, b, L, c0, lane, active, sb[r]);
#pragma unroll
      for (int i = 0; i < CPL * SW; i++) {
        const float v = ldf(H, row * S + (size_t)cc * SW + i);
        hc[r][i] = k >= 2 ? v : 0.f;  // sweep 1 starts from h = 0
      }
#pragma unroll
      for (int c = 0; c < CPL; c++)
#pragma unroll
        for (int i = 0; i < AW; i++) pg[r][c][i] = pagg[((size_t)L * CH + lane * CPL + c) * AW + i];
    }
#pragma unroll
    for (int r = 0; r < R; r++) {
      const int j = jc + r, L = stripe * nt + j;
      if (!(active && j < j1)) continue;
#pragma unroll
      for (int c = 0; c < CPL; c++) {
        float f[SW], J[SW * SW];
        chan_cell<CELL>(&sb[r][c * SW], u[r][c], w[c], f, J);
        Op<SW> e, p;
#pragma unroll
        for (int i = 0; i < SW * SW; i++) {
          e.A[i] = J[i];
          p.A[i] = pg[r][c][i];
        }
#pragma unroll
        for (int i = 0; i < SW; i++) {
          e.b[i] = f[i] - hc[r][c * SW + i];
          p.b[i] = pg[r][c][SW * SW + i];
        }
        const Op<SW> full = compose(p, e);
        float *pa = pagg + ((size_t)L * CH + lane * CPL + c) * AW;
#pragma unroll
        for (int i = 0; i < SW * SW; i++) pa[i] = full.A[i];
#pragma unroll
        for (int i = 0; i < SW; i++) pa[SW * SW + i] = full.b[i];
        tot[c] = compose(full, tot[c]);
      }
    }
  }
#pragma unroll
  for (int c = 0; c < CPL; c++) {
#pragma unroll
    for (int i = 0; i < SW * SW; i++) s_tot[wid][lane * CPL + c][i] = tot[c].A[i];
#pragma unroll
    for (int i = 0; i < SW; i++) s_tot[wid][lane * CPL + c][SW * SW + i] = tot[c].b[i];
  }
  __syncthreads();
  float cur[CPL][SW];
#pragma unroll
  for (int c = 0; c < CPL; c++) {
#pragma unroll
    for (int i = 0; i < SW; i++) cur[c][i] = 0.f;
    for (int v = 0; v < wid; v++) {
      Op<SW> o;
      const float *q = s_tot[v][lane * CPL + c];
#pragma unroll
      for (int i = 0; i < SW * SW; i++) o.A[i] = q[i];
#pragma unroll
      for (int i = 0; i < SW; i++) o.b[i] = q[SW * SW + i];
      float y[SW];
      op_apply(o, cur[c], y);
#pragma unroll
      for (int i = 0; i < SW; i++) cur[c][i] = y[i];
    }
  }
  if (!active) return;
  for (int jc = j0; jc < j1; jc += R) {
    float pg[R][CPL][AW];
#pragma unroll
    for (int r = 0; r < R; r++) {
      const int L = stripe * nt + (jc + r < j1 ? jc + r : j0);
#pragma unroll
      for (int c = 0; c < CPL; c++)
#pragma unroll
        for (int i = 0; i < AW; i++) pg[r][c][i] = pagg[((size_t)L * CH + lane * CPL + c) * AW + i];
    }
#pragma unroll
    for (int r = 0; r < R; r++) {
      const int j = jc + r, L = stripe * nt + j;
      if (j >= j1) continue;
#pragma unroll
      for (int c = 0; c < CPL; c++) {
        float *cp = carry + ((size_t)L * CH + lane * CPL + c) * SW;
#pragma unroll
        for (int i = 0; i < SW; i++) cp[i] = cur[c][i];
        Op<SW> o;
#pragma unroll
        for (int i = 0; i < SW * SW; i++) o.A[i] = pg[r][c][i];
#pragma unroll
        for (int i = 0; i < SW; i++) o.b[i] = pg[r][c][SW * SW + i];
        float y[SW];
        op_apply(o, cur[c], y);
#pragma unroll
        for (int i = 0; i < SW; i++) cur[c][i] = y[i];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Adjoint as streaming passes.  With mu_t = J_t^T lambda_t, the reverse
// recurrence lambda_t = g_t + J_{t+1}^T lambda_{t+1} (lambda past the last
// step is 0) becomes mu_t = J_t^T mu_{t+1} + J_t^T g_t, whose element at step
// t needs only that step's inputs (h_{t-1}, U_t, g_t) -- the same ones the
// cell's vector-Jacobian product at step t takes, which returns mu_t itself.
//   k_chan_adj_pass<false>  each wavefront composes its tile's elements, top
//                           step first, into the tile aggregate;
//   k_chan_adj_carry        reverse exclusive scan: mu entering each tile
//                           from the tile above (0 for the last tile);
//   k_chan_adj_pass<true>   each wavefront walks its tile downwards from its
//                           carry: lambda_t = g_t + mu_{t+1}, then the
//                           cell's VJP gives mu_t, dU_t and the weight
//                           partials; stores lambda, dU and dh0 = mu_0.
// ---------------------------------------------------------------------------
template <int CELL, typename ST, int CPL, bool APPLY>
__global__ __launch_bounds__(256) void k_chan_adj_pass(const ChanArgs a) {
  constexpr int SW = cell_code(CELL) == C_LSTM ? 2 : 1, CH = 64 * CPL, AW = SW * SW + SW, ES = (int)sizeof(ST);
  constexpr int UW = words_of<ST, CPL>(), HW = words_of<ST, CPL * SW>(), TT = CHAN2_TT;
  const int lane = threadIdx.x & 63, wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tile = blockIdx.x * 4 + wid;
  if (tile >= a.ntiles) return;
  const int T = a.T, n = a.n, S = SW * n;
  const int j = tile / a.stripes, stripe = tile % a.stripes;
  const int CG = (n + CH - 1) / CH, b = stripe / CG;
  const int c0 = (stripe % CG) * CH + lane * CPL;
  const bool active = c0 < n;
  const int L = stripe * a.tps + j, t0 = j * TT, nrows = min(TT, T - t0);
  const unsigned lane_oob = active ? 0u : SC_OOB;
  // lane parts of the offsets with the idle bit, formed once (see k_chan_pass)
  const unsigned ulane = (unsigned)(c0 * ES) | lane_oob, slane = (unsigned)(c0 * SW * ES) | lane_oob;
  ChanW w[CPL];
#pragma unroll
  for (int c = 0; c < CPL; c++) w[c] = load_chan_w<ST, CELL>(a, active ? c0 + c : 0);

  // rows of the tile: U_t and g_t at [t0, t0 + nrows); h_{t-1} from the row
  // before (the first tile's step 0 takes h0 instead: its row offset is -1,
  // outside the resource)
  const size_t row0 = (size_t)b * T + t0;
  const int hsh = t0 > 0 ? 0 : 1;  // h row of step s is s - hsh
  const Rsrc ru = sc_rsrc((const ST *)a.U + row0 * 3 * n, (unsigned)(nrows * 3 * n * ES));
  const Rsrc rg = sc_rsrc((const ST *)a.g + row0 * S, (unsigned)(nrows * S * ES));
  const Rsrc rh = sc_rsrc((const ST *)a.h + (row0 - 1 + hsh) * S, (unsigned)((nrows - hsh) * S * ES));
  float h0v[CPL * SW];
  {
    const ST *hp = (t0 == 0 && a.h0) ? (const ST *)a.h0 + (size_t)b * S + (size_t)(active ? c0 : 0) * SW
                                     : (const ST *)a.Wh;
#pragma unroll
    for (int i = 0; i < CPL * SW; i++) {
      const float v = ldf(hp, i);
      h0v[i] = (t0 == 0 && a.h0) ? v : 0.f;
    }
  }
  float mu[CPL * SW];
  Op<SW> agg[CPL];
  float acc[CPL][CHAN_P];
#pragma unroll
  for (int c = 0; c < CPL; c++) {
    agg[c] = op_identity<SW>();
#pragma unroll
    for (int p = 0; p < CHAN_P; p++) acc[c][p] = 0.f;
  }
#pragma unroll
  for (int i = 0; i < CPL * SW; i++) mu[i] = 0.f;
  if constexpr (APPLY) {
    const float *cp = (const float *)a.incl + ((size_t)L * CH + lane * CPL) * SW;
#pragma unroll
    for (int i = 0; i < CPL * SW; i++) mu[i] = cp[i];
  }
  const Rsrc rl = sc_rsrc(APPLY && a.lam ? (ST *)a.lam + row0 * S : nullptr, (unsigned)(nrows * S * ES));
  const Rsrc rd = sc_rsrc(APPLY ? (ST *)a.dU + row0 * 3 * n : nullptr, (unsigned)(nrows * 3 * n * ES));

  unsigned ua[C2_P][3][UW], ha[C2_P][HW], ga[C2_P][HW], ub[C2_P][3][UW], hb[C2_P][HW], gb[C2_P][HW];
  // group gi holds steps s = TT - 1 - (gi * C2_P + q), top step first
  auto load = [&](int gi, unsigned (&u)[C2_P][3][UW], unsigned (&h)[C2_P][HW], unsigned (&g)[C2_P][HW]) {
#pragma unroll
    for (int q = 0; q < C2_P; q++) {
      const int s = TT - 1 - (gi * C2_P + q);  // negative past the tile: outside every resource
#pragma unroll
      for (int k3 = 0; k3 < 3; k3++) bldw<CPL * ES>(ru, ulane + (unsigned)((s * 3 * n + k3 * n) * ES), u[q][k3]);
      bldw<CPL * SW * ES>(rh, slane + (unsigned)((s - hsh) * S * ES), h[q]);
      bldw<CPL * SW * ES>(rg, slane + (unsigned)(s * S * ES), g[q]);
    }
  };
  auto steps = [&](int gi, const unsigned (&u)[C2_P][3][UW], const unsigned (&h)[C2_P][HW],
                   const unsigned (&g)[C2_P][HW]) {
#pragma unroll
    for (int q = 0; q < C2_P; q++) {
      const int s = TT - 1 - (gi * C2_P + q);
      const bool valid = active && s < nrows;
      float lo[CPL * SW], du[3][CPL], dso[CPL * SW];
#pragma unroll
      for (int c = 0; c < CPL; c++) {
        const float uc[3] = {unpackw<ST>(u[q][0], c), unpackw<ST>(u[q][1], c), unpackw<ST>(u[q][2], c)};
        float sp[SW], gc[SW];
#pragma unroll
        for (int i = 0; i < SW; i++) {
          const float hv = unpackw<ST>(h[q], c * SW + i);
          sp[i] = (t0 + s == 0) ? h0v[c * SW + i] : hv;
          gc[i] = unpackw<ST>(g[q], c * SW + i);
        }
        if constexpr (!APPLY) {
          // element (J^T, J^T g) of mu's recurrence, composed after the steps above
          float f[SW], J[SW * SW];
          chan_cell<CELL>(sp, uc, w[c], f, J);
          Op<SW> e;
#pragma unroll
          for (int r = 0; r < SW; r++) {
            float v = 0.f;
#pragma unroll
            for (int q2 = 0; q2 < SW; q2++) {
              e.A[r * SW + q2] = valid ? J[q2 * SW + r] : (r == q2 ? 1.f : 0.f);
              v = fmaf(J[q2 * SW + r], gc[q2], v);
            }
            e.b[r] = valid ? v : 0.f;
          }
          agg[c] = compose(e, agg[c]);
        } else {
          float lam[SW], ds[SW], dU[3], tacc[CHAN_P];
#pragma unroll
          for (int i = 0; i < SW; i++) lam[i] = gc[i] + mu[c * SW + i];
#pragma unroll
          for (int p = 0; p < CHAN_P; p++) tacc[p] = 0.f;
          chan_cell_vjp<CELL>(sp, uc, lam, w[c], ds, dU, tacc);
          tacc[8] += dU[0];
          tacc[9] += dU[1];
          tacc[10] += dU[2];
#pragma unroll
          for (int p = 0; p < CHAN_P; p++) acc[c][p] += valid ? tacc[p] : 0.f;
#pragma unroll
          for (int i = 0; i < SW; i++) {
            mu[c * SW + i] = valid ? ds[i] : mu[c * SW + i];
            lo[c * SW + i] = lam[i];
            dso[c * SW + i] = ds[i];
          }
#pragma unroll
          for (int k3 = 0; k3 < 3; k3++) du[k3][c] = dU[k3];
        }
      }
      if constexpr (APPLY) {
        bst<ST, CPL * SW, SC_NT>(rl, slane + (unsigned)(s * S * ES), lo);
#pragma unroll
        for (int k3 = 0; k3 < 3; k3++) bst<ST, CPL>(rd, ulane + (unsigned)((s * 3 * n + k3 * n) * ES), du[k3]);
        if (t0 + s == 0 && a.dh0 && active) {
#pragma unroll
          for (int i = 0; i < CPL * SW; i++) stf((ST *)a.dh0 + (size_t)b * S + (size_t)c0 * SW + i, 0, dso[i]);
        }
      }
    }
  };
  load(0, ua, ha, ga);
  for (int gi = 0; gi < C2_NG; gi += 2) {
    load(gi + 1, ub, hb, gb);
    steps(gi, ua, ha, ga);
    load(gi + 2, ua, ha, ga);
    steps(gi + 1, ub, hb, gb);
  }
  if (!active) return;
  if constexpr (!APPLY) {
    float *pa = (float *)a.agg + ((size_t)L * CH + lane * CPL) * AW;
#pragma unroll
    for (int c = 0; c < CPL; c++) {
#pragma unroll
      for (int i = 0; i < SW * SW; i++) pa[c * AW + i] = agg[c].A[i];
#pragma unroll
      for (int i = 0; i < SW; i++) pa[c * AW + SW * SW + i] = agg[c].b[i];
    }
  } else {
    float *pp = a.part + ((size_t)L * CH + lane * CPL) * CHAN_P;
#pragma unroll
    for (int c = 0; c < CPL; c++)
#pragma unroll
      for (int p = 0; p < CHAN_P; p++) pp[c * CHAN_P + p] = acc[c][p];
  }
}

// Reverse exclusive scan of the tile aggregates of one stripe (block): mu
// entering each tile from the tile above, C2_CW wavefronts over contiguous
// ranges of tiles (loads of C2_R tiles issued together).  FUSED: the last
// sweep's pass composed each tile's steps but its first (see k_chan_pass);
// that step's element, at the final state before the tile, is composed here
// first and the full aggregate written back.
template <int CELL, typename ST, int CPL, bool FUSED>
__global__ __launch_bounds__(64 * C2_CW) void k_chan_adj_carry(const ChanArgs a) {
  constexpr int SW = cell_code(CELL) == C_LSTM ? 2 : 1;
  constexpr int CH = 64 * CPL, AW = SW * SW + SW, R = C2_R, TT = CHAN2_TT;
  __shared__ float s_tot[C2_CW][CH][AW];
  const int lane = threadIdx.x & 63, wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int stripe = blockIdx.x, nt = a.tps, per = (nt + C2_CW - 1) / C2_CW;
  // wavefront wid takes the wid-th range from the top
  const int j1 = max(0, nt - wid * per), j0 = max(0, j1 - per);
  float *carry = (float *)a.incl;
  if constexpr (FUSED) {
    const int T = a.T, n = a.n, S = SW * n;
    const int CG = (n + CH - 1) / CH, b = stripe / CG;
    const int c0 = (stripe % CG) * CH + lane * CPL;
    const bool active = c0 < n;
    const int cc = active ? c0 : 0;
    ChanW w[CPL];
#pragma unroll
    for (int c = 0; c < CPL; c++) w[c] = load_chan_w<ST, CELL>(a, cc + c);
    const ST *U = (const ST *)a.U, *H = (const ST *)a.h, *G = (const ST *)a.g;
    float *pagg = (float *)a.agg;
    for (int jc = j0; jc < j1; jc += R) {
      // every load of the chunk is issued unconditionally (idle slots read a
      // valid tile's data and are discarded), then used
      float u[R][CPL][3], sb[R][CPL * SW], gv[R][CPL * SW], pg[R][CPL][AW];
#pragma unroll
      for (int r = 0; r < R; r++) {
        const int jj = jc + r < j1 ? jc + r : j0, L = stripe * nt + jj, t0 = jj * TT;
        const size_t row = (size_t)b * T + t0;
        // the final state before step t0: h[t0 - 1], h0 or 0
        const ST *hp = t0 > 0 ? H + (row - 1) * S + (size_t)cc * SW
                              : (a.h0 ? (const ST *)a.h0 + (size_t)b * S + (size_t)cc * SW : H);
#pragma unroll
        for (int c = 0; c < CPL; c++)
#pragma unroll
          for (int gi = 0; gi < 3; gi++) u[r][c][gi] = ldf(U, row * 3 * n + (size_t)gi * n + cc + c);
#pragma unroll
        for (int i = 0; i < CPL * SW; i++) {
          const float v = ldf(hp, i);
          sb[r][i] = (t0 > 0 || a.h0) ? v : 0.f;
          gv[r][i] = ldf(G, row * S + (size_t)cc * SW + i);
        }
#pragma unroll
        for (int c = 0; c < CPL; c++)
#pragma unroll
          for (int i = 0; i < AW; i++) pg[r][c][i] = pagg[((size_t)L * CH + lane * CPL + c) * AW + i];
      }
#pragma unroll
      for (int r = 0; r < R; r++) {
        const int j = jc + r, L = stripe * nt + j;
        if (!(active && j < j1)) continue;
#pragma unroll
        for (int c = 0; c < CPL; c++) {
          float f[SW], J[SW * SW];
          chan_cell<cell_code(CELL)>(&sb[r][c * SW], u[r][c], w[c], f, J);
          Op<SW> e, p;
#pragma unroll
          for (int q = 0; q < SW; q++) {
            float v = 0.f;
#pragma unroll
            for (int q2 = 0; q2 < SW; q2++) {
              e.A[q * SW + q2] = J[q2 * SW + q];
              v = fmaf(J[q2 * SW + q], gv[r][c * SW + q2], v);
            }
            e.b[q] = v;
          }
#pragma unroll
          for (int i = 0; i < SW * SW; i++) p.A[i] = pg[r][c][i];
#pragma unroll
          for (int i = 0; i < SW; i++) p.b[i] = pg[r][c][SW * SW + i];
          const Op<SW> full = compose(e, p);  // the first step acts last
          float *pa = pagg + ((size_t)L * CH + lane * CPL + c) * AW;
#pragma unroll
          for (int i = 0; i < SW * SW; i++) pa[i] = full.A[i];
#pragma unroll
          for (int i = 0; i < SW; i++) pa[SW * SW + i] = full.b[i];
        }
      }
    }
  }
  const float *pagg = (const float *)a.agg;
  auto ld_op = [&](int j, int c) {
    Op<SW> o;
    const float *q = pagg + (((size_t)stripe * nt + j) * CH + lane * CPL + c) * AW;
#pragma unroll
    for (int i = 0; i < SW * SW; i++) o.A[i] = q[i];
#pragma unroll
    for (int i = 0; i < SW; i++) o.b[i] = q[SW * SW + i];
    return o;
  };
  Op<SW> tot[CPL];
#pragma unroll
  for (int c = 0; c < CPL; c++) tot[c] = op_identity<SW>();
  for (int jc = j1 - 1; jc >= j0; jc -= R) {  // top tile of the range first
    Op<SW> o[R][CPL];
#pragma unroll
    for (int r = 0; r < R; r++)
#pragma unroll
      for (int c = 0; c < CPL; c++) o[r][c] = ld_op(jc - r >= j0 ? jc - r : j0, c);
#pragma unroll
    for (int r = 0; r < R; r++)
#pragma unroll
      for (int c = 0; c < CPL; c++)
        if (jc - r >= j0) tot[c] = compose(o[r][c], tot[c]);
  }
#pragma unroll
  for (int c = 0; c < CPL; c++) {
#pragma unroll
    for (int i = 0; i < SW * SW; i++) s_tot[wid][lane * CPL + c][i] = tot[c].A[i];
#pragma unroll
    for (int i = 0; i < SW; i++) s_tot[wid][lane * CPL + c][SW * SW + i] = tot[c].b[i];
  }
  __syncthreads();
  float cur[CPL][SW];
#pragma unroll
  for (int c = 0; c < CPL; c++) {
#pragma unroll
    for (int i = 0; i < SW; i++) cur[c][i] = 0.f;
    for (int v = 0; v < wid; v++) {  // ranges above this one, top first
      Op<SW> o;
      const float *q = s_tot[v][lane * CPL + c];
#pragma unroll
      for (int i = 0; i < SW * SW; i++) o.A[i] = q[i];
#pragma unroll
      for (int i = 0; i < SW; i++) o.b[i] = q[SW * SW + i];
      float y[SW];
      op_apply(o, cur[c], y);
#pragma unroll
      for (int i = 0; i < SW; i++) cur[c][i] = y[i];
    }
  }
  for (int jc = j1 - 1; jc >= j0; jc -= R) {
    Op<SW> o[R][CPL];
#pragma unroll
    for (int r = 0; r < R; r++)
#pragma unroll
      for (int c = 0; c < CPL; c++) o[r][c] = ld_op(jc - r >= j0 ? jc - r : j0, c);
#pragma unroll
    for (int r = 0; r < R; r++) {
      const int jj = jc - r;
      if (jj < j0) continue;
#pragma unroll
      for (int c = 0; c < CPL; c++) {
        float *cp = carry + (((size_t)stripe * nt + jj) * CH + lane * CPL + c) * SW;
#pragma unroll
        for (int i = 0; i < SW; i++) cp[i] = cur[c][i];
        float y[SW];
        op_apply(o[r][c], cur[c], y);
#pragma unroll
        for (int i = 0; i < SW; i++) cur[c][i] = y[i];
      }
    }
  }
}

template <int CELL, typename ST, int CPL>
static hipError_t chan2_adj_launch(const ChanArgs &a, bool fused, hipStream_t s) {
  const unsigned grid = (unsigned)((a.ntiles + 3) / 4);
  if (fused) {
    hipLaunchKernelGGL((k_chan_adj_carry<CELL, ST, CPL, true>), dim3(a.stripes), dim3(64 * C2_CW), 0, s, a);
  } else {
    hipLaunchKernelGGL((k_chan_adj_pass<CELL, ST, CPL, false>), dim3(grid), dim3(256), 0, s, a);
    hipLaunchKernelGGL((k_chan_adj_carry<CELL, ST, CPL, false>), dim3(a.stripes), dim3(64 * C2_CW), 0, s, a);
  }
  hipLaunchKernelGGL((k_chan_adj_pass<CELL, ST, CPL, true>), dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_chan2_adjoint(int cell, bool bf16, const ChanArgs &a, hipStream_t s, bool fused) {
  const ChanGeomInfo g = chan2_geom(cell, a.n);
  if (cell == C_GRU_DIAG) {
    if (g.CPL == 2)
      return bf16 ? chan2_adj_launch<C_GRU_DIAG, uint16_t, 2>(a, fused, s)
                  : chan2_adj_launch<C_GRU_DIAG, float, 2>(a, fused, s);
    return bf16 ? chan2_adj_launch<C_GRU_DIAG, uint16_t, 1>(a, fused, s)
                : chan2_adj_launch<C_GRU_DIAG, float, 1>(a, fused, s);
  }
  if (cell == C_LSTM)
    return bf16 ? chan2_adj_launch<C_LSTM, uint16_t, 1>(a, fused, s) : chan2_adj_launch<C_LSTM, float, 1>(a, fused, s);
  return hipErrorInvalidValue;
}

ChanGeomInfo chan2_geom(int cell, int n) {
  ChanGeomInfo g;
  g.CPL = (cell == C_GRU_DIAG && n % 2 == 0) ? 2 : 1;
  g.TW = CHAN2_TT;
  g.CH = 64 * g.CPL;
  g.TT = CHAN2_TT;
  return g;
}

template <int CELL, typename ST, int CPL>
static hipError_t chan2_launch(const ChanArgs &a, int what, hipStream_t s) {
  const unsigned pass_grid = (unsigned)((a.ntiles + 3) / 4);
  switch (what) {
    case CHAN2_FIRST:
      hipLaunchKernelGGL((k_chan_pass<CELL, ST, CPL, false, true>), dim3(pass_grid), dim3(256), 0, s, a);
      break;
    case CHAN2_CARRY:
      hipLaunchKernelGGL((k_chan_carry<CELL, ST, CPL>), dim3(a.stripes), dim3(64 * C2_CW), 0, s, a);
      break;
    case CHAN2_APPLY_NEXT:
      hipLaunchKernelGGL((k_chan_pass<CELL, ST, CPL, true, true>), dim3(pass_grid), dim3(256), 0, s, a);
      break;
    case CHAN2_APPLY:
      hipLaunchKernelGGL((k_chan_pass<CELL, ST, CPL, true, false>), dim3(pass_grid), dim3(256), 0, s, a);
      break;
    case CHAN2_APPLY_ADJ:
      hipLaunchKernelGGL((k_chan_pass<CELL, ST, CPL, true, false, true>), dim3(pass_grid), dim3(256), 0, s, a);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int CELL>
static hipError_t chan2_dtype(bool bf16, int CPL, const ChanArgs &a, int what, hipStream_t s) {
  if constexpr (cell_code(CELL) == C_GRU_DIAG) {
    if (CPL == 2) return bf16 ? chan2_launch<CELL, uint16_t, 2>(a, what, s) : chan2_launch<CELL, float, 2>(a, what, s);
  }
  return bf16 ? chan2_launch<CELL, uint16_t, 1>(a, what, s) : chan2_launch<CELL, float, 1>(a, what, s);
}

hipError_t launch_chan2(int cell, int apx, bool bf16, const ChanArgs &a, int what, hipStream_t s) {
  const int CPL = chan2_geom(cell, a.n).CPL;
  if (cell == C_GRU_DIAG) {  // its Jacobian is diagonal: the diagonal approximation is exact
    if (apx == APX_NEWTON || apx == APX_DIAG) return chan2_dtype<C_GRU_DIAG>(bf16, CPL, a, what, s);
    if (apx == APX_ZERO) return chan2_dtype<C_GRU_DIAG + 16 * APX_ZERO>(bf16, CPL, a, what, s);
  } else if (cell == C_LSTM) {
    if (apx == APX_NEWTON) return chan2_dtype<C_LSTM>(bf16, CPL, a, what, s);
    if (apx == APX_DIAG) return chan2_dtype<C_LSTM + 16 * APX_DIAG>(bf16, CPL, a, what, s);
    if (apx == APX_ZERO) return chan2_dtype<C_LSTM + 16 * APX_ZERO>(bf16, CPL, a, what, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace pr

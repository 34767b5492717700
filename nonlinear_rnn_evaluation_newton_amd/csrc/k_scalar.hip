// Scalar-state Newton sweep (n = 1, d = 1), the shape of DEER's headline
// measurement ("Parallelizing non-linear sequential models over the sequence
// length", Experiments: GRU with batch 16 and 2^20 steps).  Same algorithm
// as the generic time-parallel sweep -- cell, Jacobian and residual at every
// step, affine scan of (J_t, r_t), in-place update, convergence measure --
// written so that a step costs about forty VALU instructions and the memory
// system never idles:
//  * the cell's weights are folded once per solve into a coefficient table
//    (exp2 scale factors included) read through the scalar cache;
//  * each lane owns 4 consecutive steps per group (16-byte loads and
//    stores), 2 groups per wavefront, 7 compute wavefronts per tile;
//  * two register sets alternate between tiles: the loads of the block's
//    next tile are issued before the current tile is computed, so HBM
//    streams while the VALU works and while the look-back waits;
//  * the wavefront scan runs on DPP-fused multiply/FMA instructions (lanes
//    whose source falls outside the pattern keep their value, which is the
//    identity of the composition);
//  * a lane's entering state comes from its neighbour's exit state by one
//    DPP shift in the update phase;
//  * full tiles are compiled without per-step bounds selects.
#include "k_time_impl.h"

namespace pr {

#ifndef SC_QDEF
#define SC_QDEF 2
#endif
constexpr int SC_V = 4, SC_Q = SC_QDEF;
constexpr int SC_CW = 7;                       // compute wavefronts per block
constexpr int SC_WSTEPS = SC_Q * 64 * SC_V;    // steps per compute wavefront
constexpr int SC_TILE = SC_CW * SC_WSTEPS;     // steps per tile
constexpr int SC_THREADS = 64 * (SC_CW + 1);   // + the look-back wavefront (a multiple of 4 wavefronts)
constexpr int SC_LB = SC_CW;                   // wavefront id of the look-back wavefront
constexpr float LOG2E = 1.4426950408889634f;

// Coefficient table (16 floats) derived from the weights once per solve.
// GRU (gate rows r, z, n of W_x [3,1], W_h [3,1], b_x [3], b_h [3]):
//  0..2  -log2e * (w_xr, w_hr, b_xr + b_hr)      -> exp2 argument of sigm(a_r)
//  3..5  -log2e * (w_xz, w_hz, b_xz + b_hz)
//  6..7  2 log2e * (w_xn, b_xn)                  -> 2 log2e * U_n
//  8..9  2 log2e * (w_hn, b_hn)                  -> 2 log2e * q
//  10    w_hz, 11 w_hn, 12 w_hr / (2 log2e)      -> Jacobian
// tanh RNN / linear: 0 w_x, 1 w_h, 2 b_x + b_h.
__global__ void k_scalar_coef(const float *Wx, const float *bx, const float *Wh, const float *bh, int cell,
                              float *coef) {
  if (threadIdx.x != 0) return;
  auto B = [&](const float *p, int i) { return p ? p[i] : 0.f; };
  for (int i = 0; i < 16; i++) coef[i] = 0.f;
  if (cell == C_GRU) {
    coef[0] = -LOG2E * Wx[0]; coef[1] = -LOG2E * Wh[0]; coef[2] = -LOG2E * (B(bx, 0) + B(bh, 0));
    coef[3] = -LOG2E * Wx[1]; coef[4] = -LOG2E * Wh[1]; coef[5] = -LOG2E * (B(bx, 1) + B(bh, 1));
    coef[6] = 2.f * LOG2E * Wx[2]; coef[7] = 2.f * LOG2E * B(bx, 2);
    coef[8] = 2.f * LOG2E * Wh[2]; coef[9] = 2.f * LOG2E * B(bh, 2);
    coef[10] = Wh[1]; coef[11] = Wh[2]; coef[12] = Wh[0] / (2.f * LOG2E);
  } else {
    coef[0] = Wx[0]; coef[1] = Wh[0]; coef[2] = B(bx, 0) + B(bh, 0);
  }
}

// f and J of the scalar cell at state s, input x.
template <int CELL>
__device__ inline void scalar_cell(const float *__restrict__ C, float s, float x, float &f, float &J) {
  if constexpr (CELL == C_GRU) {
    const float er = __builtin_amdgcn_exp2f(fmaf(C[0], x, fmaf(C[1], s, C[2])));
    const float ez = __builtin_amdgcn_exp2f(fmaf(C[3], x, fmaf(C[4], s, C[5])));
    const float r = __builtin_amdgcn_rcpf(1.f + er);
    const float z = __builtin_amdgcn_rcpf(1.f + ez);
    const float q2 = fmaf(C[8], s, C[9]);  // 2 log2e q
    const float ec = __builtin_amdgcn_exp2f(fmaf(r, q2, fmaf(C[6], x, C[7])));
    const float c = fmaf(-2.f, __builtin_amdgcn_rcpf(1.f + ec), 1.f);
    const float sc = s - c;
    f = fmaf(z, sc, c);
    const float zz = fmaf(-z, z, z);    // z (1 - z)
    const float cc = fmaf(-c, c, 1.f);  // 1 - c^2
    const float e2 = fmaf(-z, cc, cc);  // (1 - z)(1 - c^2)
    const float rr = fmaf(-r, r, r);    // r (1 - r)
    const float inner = fmaf(q2 * C[12], rr, r * C[11]);  // r w_hn + q r (1 - r) w_hr
    J = fmaf(e2, inner, fmaf(sc * zz, C[10], z));
  } else if constexpr (CELL == C_TANH) {
    const float e = __builtin_amdgcn_exp2f(2.f * LOG2E * fmaf(C[0], x, fmaf(C[1], s, C[2])));
    f = fmaf(-2.f, __builtin_amdgcn_rcpf(1.f + e), 1.f);
    J = fmaf(-f, f, 1.f) * C[1];
  } else {
    f = fmaf(C[0], x, fmaf(C[1], s, C[2]));
    J = C[1];
  }
}

// Inclusive scan of scalar affine maps (A, b) across the wavefront in lane
// order: after it, lane l holds op_l o ... o op_0.  Each level composes a
// lane with the lane the DPP pattern names (b += A * b_src, then
// A *= A_src); lanes with no source are not written, i.e. composed with the
// identity.  Two wait states precede every DPP read of a VGPR written by
// the previous VALU instruction.  Requires all 64 lanes active.
__device__ inline void wave_scan_affine1(float &A, float &b) {
  asm volatile(
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %1, %1, %0 row_shr:1 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_mul_f32_dpp %0, %0, %0 row_shr:1 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %1, %1, %0 row_shr:2 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_mul_f32_dpp %0, %0, %0 row_shr:2 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %1, %1, %0 row_shr:4 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_mul_f32_dpp %0, %0, %0 row_shr:4 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %1, %1, %0 row_shr:8 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_mul_f32_dpp %0, %0, %0 row_shr:8 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %1, %1, %0 row_bcast:15 row_mask:0xa bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_mul_f32_dpp %0, %0, %0 row_bcast:15 row_mask:0xa bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %1, %1, %0 row_bcast:31 row_mask:0xc bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_mul_f32_dpp %0, %0, %0 row_bcast:31 row_mask:0xc bank_mask:0xf\n\t"
      "s_nop 1"
      : "+v"(A), "+v"(b));
}

__device__ inline float rdlane(float v, int l) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l)); }

// lane l receives v of lane l - 1; lane 0 receives first
__device__ inline float shift_in(float first, float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(first), __float_as_int(v), 0x138, 0xf, 0xf, false));
}

// Memory access of the sweep goes through buffer instructions on per-row
// buffer resources: the hardware range check returns zero for loads past the
// end of a row and drops stores past it (and at offset SC_OOB), so every
// load and store in the tile loop is unconditional.  That keeps the
// compiler's count of memory operations in flight exact: loads and stores
// share one in-order counter on this architecture, and a memory instruction
// under a branch would make later waits conservative, draining recent
// stores before the prefetched data can be used.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr unsigned SC_OOB = 0x80000000u;  // offset beyond every resource: load 0, store dropped
constexpr int SC_SC1 = 16;                // cache policy: device-scope coherent access

__device__ inline Rsrc sc_rsrc(const void *base, unsigned bytes) {
  // raw buffer, stride 0, 32-bit data format in the fourth descriptor word
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}
__device__ inline float4 ld4(Rsrc r, unsigned off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w));
}
__device__ inline float ld1(Rsrc r, unsigned off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ inline void st4(Rsrc r, unsigned off, float a, float b, float c, float d) {
  u32x4 v;
  v.x = __float_as_uint(a); v.y = __float_as_uint(b); v.z = __float_as_uint(c); v.w = __float_as_uint(d);
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 0);
}
__device__ inline void st1(Rsrc r, unsigned off, float a) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(a), r, off, 0, 0);
}

// Raw inputs of one tile for one thread: x and the current iterate h for its
// groups, and (lane 0's) state before the wavefront's first step.
struct ScRaw {
  float4 x[SC_Q], h[SC_Q];
  float sw;
};

// Issue the loads of tile `id`.  Needs T % 4 == 0, so a lane's 4 steps are all
// inside or all outside [0, T).  In the first sweep the iterate is the zero
// guess and h is not read.
template <bool FIRST>
__device__ inline void sc_load(const TimeArgs &a, int id, ScRaw &R) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, k = a.k, B = a.B, T = a.T;
  const int j = id / B, b = id % B;
  const int t0 = j * SC_TILE + wid * SC_WSTEPS;
  const Rsrc rx = sc_rsrc(a.x + (size_t)b * T, (unsigned)T * 4u);
  const Rsrc rh = sc_rsrc(a.h + (size_t)b * T, (unsigned)T * 4u);
#pragma unroll
  for (int q = 0; q < SC_Q; q++) {
    const unsigned off = (unsigned)(t0 + (q * 64 + lane) * SC_V) * 4u;
    R.x[q] = ld4(rx, off);
    if (!FIRST) R.h[q] = ld4(rh, off);
  }
  // the state before step t0: h0 (t0 = 0; zero without h0), the predecessor
  // tile's last state from the previous sweep (wavefront 0), or h[t0 - 1],
  // which this block writes only after this load, later in this sweep.  An
  // empty resource reads zero.
  const float *sb = a.x;
  unsigned nb = 0, so = 0;
  if (t0 == 0) {
    if (a.h0) { sb = a.h0 + b; nb = 4; }
  } else if (!FIRST && t0 < T) {
    if (wid == 0) { sb = a.bnd + (size_t)((k - 1) & 1) * a.ntiles + (b * a.tiles_per_seq + j - 1); nb = 4; }
    else { sb = a.h + (size_t)b * T; nb = (unsigned)T * 4u; so = (unsigned)(t0 - 1) * 4u; }
  }
  R.sw = ld1(sc_rsrc(sb, nb), so);
}

// A computed tile waiting for its carry: per-step Jacobians, residuals and
// iterate, per-group inclusive lane scans (iA, ib) and group totals (tA, tb).
struct ScTile {
  float J[SC_Q][SC_V], R[SC_Q][SC_V], H[SC_Q][SC_V];
  float iA[SC_Q], ib[SC_Q], tA[SC_Q], tb[SC_Q];
};

// Wavefront totals of the last two computed tiles and their carries.
struct ScShared {
  float wA[2][SC_CW], wb[2][SC_CW];
  float carry[2];
  unsigned done[2];  // compute wavefronts finished with the tile in each buffer
  int stop;
  unsigned dmax[SC_CW];
};

// Descriptor resources of one sequence.
struct ScDesc {
  Rsrc agg, incl;
};
__device__ inline ScDesc sc_desc(const TimeArgs &a, int b) {
  ScDesc d;
  d.agg = sc_rsrc(a.agg + (size_t)b * a.tiles_per_seq * 2, (unsigned)a.tiles_per_seq * 16u);
  d.incl = sc_rsrc(a.incl + (size_t)b * a.tiles_per_seq, (unsigned)a.tiles_per_seq * 8u);
  return d;
}

// Cell, Jacobian and residual of every step of tile `id`, lane-serial
// composition of each lane's steps, wavefront scans, and the wavefront totals
// into LDS buffer `buf` (read after the next block barrier).
template <int CELL, bool FIRST, bool FULL>
__device__ inline void sc_compute(const TimeArgs &a, const float *C, int id, const ScRaw &R, ScTile &Tl,
                                  ScShared &sh, int buf) {
  constexpr int V = SC_V, Q = SC_Q;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, B = a.B, T = a.T;
  const int j = id / B;
  const int t0 = j * SC_TILE + wid * SC_WSTEPS;
#pragma unroll
  for (int q = 0; q < Q; q++) {
    const float xv[V] = {R.x[q].x, R.x[q].y, R.x[q].z, R.x[q].w};
    float hv[V] = {0.f, 0.f, 0.f, 0.f};
    if (!FIRST) {
      hv[0] = R.h[q].x; hv[1] = R.h[q].y; hv[2] = R.h[q].z; hv[3] = R.h[q].w;
    }
    float s = shift_in(q == 0 ? R.sw : FIRST ? 0.f : rdlane(R.h[q - 1].w, 63), hv[V - 1]);
    float A = 1.f, bb = 0.f;
    const bool in = FULL || t0 + (q * 64 + lane) * V < T;
#pragma unroll
    for (int v = 0; v < V; v++) {
      float f, Jv;
      scalar_cell<CELL>(C, s, xv[v], f, Jv);
      float rv = f - hv[v];
      if (!FULL && !in) { Jv = 1.f; rv = 0.f; }
      Tl.J[q][v] = Jv;
      Tl.R[q][v] = rv;
      Tl.H[q][v] = hv[v];
      bb = fmaf(Jv, bb, rv);
      A *= Jv;
      s = hv[v];
    }
    wave_scan_affine1(A, bb);
    Tl.iA[q] = A;
    Tl.ib[q] = bb;
    Tl.tA[q] = rdlane(A, 63);
    Tl.tb[q] = rdlane(bb, 63);
  }
  float wA = Tl.tA[0], wb = Tl.tb[0];
#pragma unroll
  for (int q = 1; q < Q; q++) {
    wb = fmaf(Tl.tA[q], wb, Tl.tb[q]);
    wA *= Tl.tA[q];
  }
  if (lane == 0) {
    sh.wA[buf][wid] = wA;
    sh.wb[buf][wid] = wb;
  }
  // The last compute wavefront to finish publishes the tile aggregate at once
  // (tile 0 of a sequence only ever publishes its inclusive prefix).  Every
  // compute wavefront executes the store; the others' offsets fall outside
  // the resource.  LDS operations of a wavefront complete in order, so the
  // totals written above are visible before its count is.
  unsigned prev = 0;
  // the totals reach LDS before the count (wait on this wavefront's LDS
  // operations; the clobber keeps the compiler from moving memory accesses
  // across)
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  if (lane == 0) prev = atomicAdd(&sh.done[buf], 1u);
  const bool last = __builtin_amdgcn_readfirstlane(prev) == SC_CW - 1;
  asm volatile("" ::: "memory");
  float tA = 1.f, tb = 0.f;
  if (last) {
#pragma unroll
    for (int w = 0; w < SC_CW; w++) {
      tb = fmaf(sh.wA[buf][w], tb, sh.wb[buf][w]);
      tA *= sh.wA[buf][w];
    }
    if (lane == 0) sh.done[buf] = 0;  // reused two tiles on, after two barriers
  }
  const ScDesc d = sc_desc(a, id % B);
  u32x4 v;
  v.x = __float_as_uint(tA); v.y = tag_agg(a.k); v.z = __float_as_uint(tb); v.w = tag_agg(a.k);
  __builtin_amdgcn_raw_buffer_store_b128(v, d.agg, (last && lane == 0 && j > 0) ? (unsigned)j * 16u : SC_OOB, 0,
                                         SC_SC1);
}

// Look-back descriptors of the 64 tiles before tile wend + 1 (lane l holds
// tile wend - 63 + l); tiles before 0 read as zero (no valid tag).
struct ScPoll {
  unsigned long long wi;  // inclusive prefix word
  u32x4 wa;               // aggregate: A bits, tag, b bits, tag
};

__device__ inline void sc_poll(Rsrc ragg, Rsrc rincl, int wend, ScPoll &P) {
  const int p = wend - 63 + (int)(threadIdx.x & 63);
  const u32x2 wi = __builtin_amdgcn_raw_buffer_load_b64(rincl, p >= 0 ? (unsigned)p * 8u : SC_OOB, 0, SC_SC1);
  P.wi = ((unsigned long long)wi.y << 32) | wi.x;
  P.wa = __builtin_amdgcn_raw_buffer_load_b128(ragg, p >= 0 ? (unsigned)p * 16u : SC_OOB, 0, SC_SC1);
}

// One look-back window (tiles wend - 63 .. wend, lane l <-> tile wend - 63 + l):
// returns 0 if a needed aggregate is not yet published, else composes the
// window into acc (acc o window) and returns 2 if the window holds an
// inclusive prefix (acc is then a constant map), 1 to continue further back.
__device__ inline int sc_window(const ScPoll &P, int wend, int k, float &accA, float &accb) {
  const int lane = threadIdx.x & 63;
  const int p = wend - 63 + lane;
  const bool hi = p >= 0 && (unsigned)(P.wi >> 32) == tag_incl(k);
  const bool ha = p >= 0 && P.wa.y == tag_agg(k) && P.wa.w == tag_agg(k);
  const unsigned long long bi = __ballot(hi);
  const int m = bi ? 63 - __clzll((long long)bi) : -1;  // nearest tile with an inclusive prefix
  const bool ok = !(lane > m && p >= 0) || ha;
  if (!__all(ok)) return 0;
  float A = 1.f, bb = 0.f;
  if (lane == m) {
    A = 0.f;
    bb = __uint_as_float((unsigned)P.wi);
  } else if (lane > m && p >= 0) {
    A = __uint_as_float(P.wa.x);
    bb = __uint_as_float(P.wa.z);
  }
  wave_scan_affine1(A, bb);
  const float wA = rdlane(A, 63), wb = rdlane(bb, 63);
  accb = fmaf(accA, wb, accb);
  accA *= wA;
  return m >= 0 ? 2 : 1;
}

// dh after the window ending at tile wend of one sequence (descriptor
// resources of that sequence), composing after acc, from descriptors polled
// earlier for that window: the decoupled look-back, re-polling while a
// needed aggregate is not yet published and stepping back while no window
// holds an inclusive prefix.
__device__ inline float sc_resolve_from(Rsrc ragg, Rsrc rincl, int wend, int k, ScPoll P, float accA, float accb,
                                        SolveState *st) {
  int spins = 0;
  int r = sc_window(P, wend, k, accA, accb);
  while (r != 2) {
    if (r == 1) {
      wend -= 64;
    } else {
      if (++spins > PR_SPIN_LIMIT) {  // the fault is reported by the host
        if ((threadIdx.x & 63) == 0) spin_fault(st);
        return 0.f;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    sc_poll(ragg, rincl, wend, P);
    r = sc_window(P, wend, k, accA, accb);
  }
  return accb;  // the composition ends in a constant map
}

// As sc_resolve, with a second, later poll of the first window to fall back on
// before re-polling.
__device__ inline float sc_resolve2(Rsrc ragg, Rsrc rincl, int j, int k, const ScPoll &P0, const ScPoll &P1,
                                    SolveState *st) {
  float accA = 1.f, accb = 0.f;
  const int r = sc_window(P0, j - 1, k, accA, accb);
  if (r == 2) return accb;
  if (r == 1) {  // the window holds no inclusive prefix yet but every aggregate: go further back
    ScPoll P;
    sc_poll(ragg, rincl, j - 65, P);
    return sc_resolve_from(ragg, rincl, j - 65, k, P, accA, accb, st);
  }
  return sc_resolve_from(ragg, rincl, j - 1, k, P1, 1.f, 0.f, st);
}

// Composition of wavefronts [0, wid) (pre) and of all four (tot) of a
// computed tile, from its LDS totals.
struct ScTot {
  float preA, preb, totA, totb;
};

__device__ inline ScTot sc_tot(const ScShared &sh, int buf, int wid) {
  ScTot r;
  r.preA = 1.f; r.preb = 0.f; r.totA = 1.f; r.totb = 0.f;
#pragma unroll
  for (int w = 0; w < SC_CW; w++) {
    const float A = sh.wA[buf][w], b = sh.wb[buf][w];
    if (w < wid) {
      r.preb = fmaf(A, r.preb, b);
      r.preA *= A;
    }
    r.totb = fmaf(A, r.totb, b);
    r.totA *= A;
  }
  return r;
}

// Look-back wavefront, for computed tile `id` whose wavefront totals are in
// LDS buffer `buf`: resolve its carry from the predecessors' descriptors,
// publish its inclusive prefix, leave the carry in LDS.  This wavefront issues no other memory operations, so its waits on
// the descriptors never queue behind the bulk loads and stores of the
// compute wavefronts.
__device__ inline void sc_lookback_tile(const TimeArgs &a, int id, ScShared &sh, int buf) {
  const int k = a.k, j = id / a.B;
  const ScTot tt = sc_tot(sh, buf, SC_CW);
  const ScDesc d = sc_desc(a, id % a.B);
  float carry = 0.f;
  if (j > 0) {
    // two polls of the same window a few hundred cycles apart: predecessors
    // of this stage publish about when this wavefront starts, and a second
    // poll already in flight costs less than a retry after the first fails
    ScPoll P0, P1;
    sc_poll(d.agg, d.incl, j - 1, P0);
    __builtin_amdgcn_s_sleep(8);
    sc_poll(d.agg, d.incl, j - 1, P1);
    carry = sc_resolve2(d.agg, d.incl, j, k, P0, P1, a.st);
  }
  u32x2 w;
  w.x = __float_as_uint(fmaf(tt.totA, carry, tt.totb));
  w.y = tag_incl(k);
  __builtin_amdgcn_raw_buffer_store_b64(w, d.incl, (threadIdx.x & 63) == 0 ? (unsigned)j * 8u : SC_OOB, 0, SC_SC1);
  if ((threadIdx.x & 63) == 0) sh.carry[buf] = carry;
}

// Update of tile `id` from its carry: the steps' new iterate, the
// convergence measure, the stores.
__device__ inline void sc_apply(const TimeArgs &a, int id, const ScTile &Tl, const ScTot &tt, const ScShared &sh,
                                int buf, unsigned &dmax) {
  constexpr int V = SC_V, Q = SC_Q;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, k = a.k, B = a.B, T = a.T;
  const int j = id / B, b = id % B, L = b * a.tiles_per_seq + j;
  const int t0 = j * SC_TILE + wid * SC_WSTEPS;
  const bool full = j * SC_TILE + SC_TILE <= T;
  float c = fmaf(tt.preA, sh.carry[buf], tt.preb);  // dh entering this wavefront's steps
  const Rsrc rh = sc_rsrc(a.h + (size_t)b * T, (unsigned)T * 4u);
  const Rsrc rb = sc_rsrc(a.bnd, (unsigned)a.ntiles * 8u);
#pragma unroll
  for (int q = 0; q < Q; q++) {
    float dh = shift_in(c, fmaf(Tl.iA[q], c, Tl.ib[q]));
    float hn[V];
#pragma unroll
    for (int v = 0; v < V; v++) {
      dh = fmaf(Tl.J[q][v], dh, Tl.R[q][v]);
      hn[v] = Tl.H[q][v] + dh;
      const unsigned u = __float_as_uint(dh) & 0x7fffffffu;
      dmax = u > dmax ? u : dmax;
    }
    st4(rh, (unsigned)(t0 + (q * 64 + lane) * V) * 4u, hn[0], hn[1], hn[2], hn[3]);  // past T: dropped
    if (q == Q - 1)  // the tile's last state, kept for the next sweep
      st1(rb, (full && wid == SC_CW - 1 && lane == 63) ? (unsigned)((k & 1) * a.ntiles + L) * 4u : SC_OOB, hn[V - 1]);
    c = fmaf(Tl.tA[q], c, Tl.tb[q]);
  }
}

template <int CELL, bool FIRST>
__device__ inline void sc_compute_any(const TimeArgs &a, const float *C, int id, const ScRaw &R, ScTile &Tl,
                                      ScShared &sh, int buf) {
  if ((id / a.B) * SC_TILE + SC_TILE <= a.T) sc_compute<CELL, FIRST, true>(a, C, id, R, Tl, sh, buf);
  else sc_compute<CELL, FIRST, false>(a, C, id, R, Tl, sh, buf);
}

// One stage of the compute wavefronts: read P's wavefront totals (LDS buffer
// bufN ^ 1; rewritten two stages on), issue the loads of the tile after N,
// compute N into buffer bufN, block barrier (the look-back wavefront has left
// P's carry), update P.
template <int CELL, bool FIRST>
__device__ inline void sc_stage(const TimeArgs &a, const float *C, int idP, const ScTile &TP, int idN,
                                const ScRaw &RN, ScRaw &Rnext, ScTile &TN, ScShared &sh, int bufN, unsigned &dmax) {
  const ScTot tt = sc_tot(sh, bufN ^ 1, threadIdx.x >> 6);
  const int nn = idN + (int)gridDim.x < a.ntiles ? idN + (int)gridDim.x : idN;  // the last reloads itself
  sc_load<FIRST>(a, nn, Rnext);
  sc_compute_any<CELL, FIRST>(a, C, idN, RN, TN, sh, bufN);
  __syncthreads();
  sc_apply(a, idP, TP, tt, sh, bufN ^ 1, dmax);
}


// Persistent grid (every block resident, grid <= tile count); block g takes
// tiles g, g + grid, ... in order.  Stage s of a block computes its tile s
// (compute wavefronts) while the look-back wavefront resolves tile s - 1; after
// the stage's barrier the compute wavefronts update tile s - 1.  Every
// look-back needs only aggregates of tiles computed in an earlier or the same
// stage of resident blocks and published before their look-backs wait, so the
// grid cannot deadlock.  The two wavefront roles run separate loops with the
// same number of barriers (tiles + 1).
template <int CELL, bool FIRST>
__global__ __launch_bounds__(SC_THREADS) void k_scalar_sweep(const TimeArgs a) {
  __shared__ ScShared sh;
  // the wavefront id through readfirstlane: the compiler then knows the role
  // branch is uniform, so each wavefront runs exactly one role's loop (and
  // its barriers) instead of both under an execution mask
  const int tid = threadIdx.x, lane = tid & 63, wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = gridDim.x, nt = a.ntiles;
  unsigned dmax = 0;
  if (wid == SC_LB) {
    if (lane == 0) {
      sh.done[0] = 0;
      sh.done[1] = 0;
    }
    if (sweep_open(a.st, a.k, a.tol, a.T, a.max_iters, &sh.stop)) return;
    __syncthreads();  // end of stage 0
    for (int id = blockIdx.x; id < nt; id += G) {
      sc_lookback_tile(a, id, sh, ((id - (int)blockIdx.x) / G) & 1);
      __syncthreads();
    }
  } else {
    // coefficients into scalar registers before any other load: a vector
    // load inside the tile loop would wait behind the prefetched tile
    float C[13];
#pragma unroll
    for (int i = 0; i < 13; i++) C[i] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(a.coef[i])));
    ScRaw R0, R1;
    ScTile T0, T1;
    int id = blockIdx.x;
    sc_load<FIRST>(a, id, R0);  // overlaps the stop check
    if (sweep_open(a.st, a.k, a.tol, a.T, a.max_iters, &sh.stop)) return;
    // stage 0: compute the first tile
    sc_load<FIRST>(a, id + G < nt ? id + G : id, R1);
    sc_compute_any<CELL, FIRST>(a, C, id, R0, T0, sh, 0);
    __syncthreads();
    int idP = id;
    id += G;
    int last = 0;  // register set of the final pending tile
    while (true) {
      if (id >= nt) { last = 0; break; }
      sc_stage<CELL, FIRST>(a, C, idP, T0, id, R1, R0, T1, sh, 1, dmax);
      idP = id;
      id += G;
      if (id >= nt) { last = 1; break; }
      sc_stage<CELL, FIRST>(a, C, idP, T1, id, R0, R1, T0, sh, 0, dmax);
      idP = id;
      id += G;
    }
    __syncthreads();  // final stage: the look-back wavefront has resolved the last tile
    const ScTot tt = sc_tot(sh, last, wid);
    if (last == 0) sc_apply(a, idP, T0, tt, sh, 0, dmax);
    else sc_apply(a, idP, T1, tt, sh, 1, dmax);
  }
  dmax = wave_max_u32(dmax);
  if (lane == 0 && wid < SC_CW) sh.dmax[wid] = dmax;
  __syncthreads();
  if (tid == 0) {
    unsigned m = sh.dmax[0];
    for (int w = 1; w < SC_CW; w++) m = sh.dmax[w] > m ? sh.dmax[w] : m;
    max_agent(&a.st->dslot[a.k & 3][blockIdx.x % PR_DSHARDS], m);
  }
}

int scalar_tile() { return SC_TILE; }

hipError_t launch_scalar_coef(const TimeArgs &a, int cell, float *coef, hipStream_t s) {
  hipLaunchKernelGGL(k_scalar_coef, dim3(1), dim3(64), 0, s, a.Wx, a.bx, a.Wh, a.bh, cell, coef);
  return hipGetLastError();
}

template <int CELL>
static hipError_t scalar_launch(const TimeArgs &a, hipStream_t s) {
  if (a.k == 1) {
    const int grid = persistent_grid<k_scalar_sweep<CELL, true>, SC_THREADS>(a.ntiles);
    if (grid <= 0) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((k_scalar_sweep<CELL, true>), dim3(grid), dim3(SC_THREADS), 0, s, a);
  } else {
    const int grid = persistent_grid<k_scalar_sweep<CELL, false>, SC_THREADS>(a.ntiles);
    if (grid <= 0) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((k_scalar_sweep<CELL, false>), dim3(grid), dim3(SC_THREADS), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_scalar_sweep(int cell, const TimeArgs &a, hipStream_t s) {
  switch (cell) {
    case C_GRU: return scalar_launch<C_GRU>(a, s);
    case C_TANH: return scalar_launch<C_TANH>(a, s);
    case C_LINEAR: return scalar_launch<C_LINEAR>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pr

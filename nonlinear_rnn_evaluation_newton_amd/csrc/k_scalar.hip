// Scalar-state kernels (n = 1, d = 1), the shape of DEER's headline
// measurement ("Parallelizing non-linear sequential models over the sequence
// length", Experiments: GRU with batch 16 and 2^20 steps): the Newton sweep
// (cell, Jacobian and residual at every step, affine scan of (J_t, r_t),
// in-place update, convergence measure) and the adjoint (reverse scan of
// (J_{t+1}, g_t) for lambda, then dx, dh0 and the weight gradients), both on
// the tile pipeline of pipe.h.  Per lane: 4 consecutive steps per group
// (16-byte accesses); the cell's weights are folded once per call into a
// coefficient table held in scalar registers; the wavefront scan runs on
// DPP-fused multiply/FMA instructions.
#include "pipe.h"

namespace pr {

constexpr int SC_V = 4;
constexpr int SC_NC = 16;  // coefficient table size
constexpr float LOG2E = 1.4426950408889634f;

// Coefficient table derived from the weights once per call.
// GRU (gate rows r, z, n of W_x [3,1], W_h [3,1], b_x [3], b_h [3]):
//  0..2  -log2e * (w_xr, w_hr, b_xr + b_hr)      -> exp2 argument of sigm(a_r)
//  3..5  -log2e * (w_xz, w_hz, b_xz + b_hz)
//  6..7  2 log2e * (w_xn, b_xn)                  -> 2 log2e * U_n
//  8..9  2 log2e * (w_hn, b_hn)                  -> 2 log2e * q
//  10    w_hz, 11 w_hn, 12 w_hr / (2 log2e)      -> Jacobian
//  13..15 w_xr, w_xz, w_xn                       -> dx
// tanh RNN / linear: 0 w_x, 1 w_h, 2 b_x + b_h.
__device__ inline void scalar_coef_fill(const float *Wx, const float *bx, const float *Wh, const float *bh, int cell,
                                        float *coef) {
  auto B = [&](const float *p, int i) { return p ? p[i] : 0.f; };
  for (int i = 0; i < SC_NC; i++) coef[i] = 0.f;
  if (cell == C_GRU) {
    coef[0] = -LOG2E * Wx[0]; coef[1] = -LOG2E * Wh[0]; coef[2] = -LOG2E * (B(bx, 0) + B(bh, 0));
    coef[3] = -LOG2E * Wx[1]; coef[4] = -LOG2E * Wh[1]; coef[5] = -LOG2E * (B(bx, 1) + B(bh, 1));
    coef[6] = 2.f * LOG2E * Wx[2]; coef[7] = 2.f * LOG2E * B(bx, 2);
    coef[8] = 2.f * LOG2E * Wh[2]; coef[9] = 2.f * LOG2E * B(bh, 2);
    coef[10] = Wh[1]; coef[11] = Wh[2]; coef[12] = Wh[0] / (2.f * LOG2E);
    coef[13] = Wx[0]; coef[14] = Wx[1]; coef[15] = Wx[2];
  } else {
    coef[0] = Wx[0]; coef[1] = Wh[0]; coef[2] = B(bx, 0) + B(bh, 0);
  }
}

// The call's workspace clearing and the coefficients in one launch (the
// coefficients lie past the cleared bytes).
__global__ void k_zero_coef(uint4 *p, size_t n16, unsigned char *tail, size_t ntail, const float *Wx,
                            const float *bx, const float *Wh, const float *bh, int cell, float *coef) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) p[i] = make_uint4(0, 0, 0, 0);
  if (blockIdx.x == 0 && threadIdx.x < ntail) tail[threadIdx.x] = 0;
  if (blockIdx.x == gridDim.x - 1 && threadIdx.x == 0) scalar_coef_fill(Wx, bx, Wh, bh, cell, coef);
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

// Reverse-mode coefficients of the scalar cell at (s, x): the derivative of f
// with respect to each pre-activation.  GRU: co = (df/da_r, df/da_z, df/da_n,
// df/dq) with q = w_hn s + b_hn; tanh / linear: co[0] = df/da.  J = df/ds.
template <int CELL>
__device__ inline void scalar_vjp(const float *__restrict__ C, float s, float x, float (&co)[4], float &J) {
  if constexpr (CELL == C_GRU) {
    const float er = __builtin_amdgcn_exp2f(fmaf(C[0], x, fmaf(C[1], s, C[2])));
    const float ez = __builtin_amdgcn_exp2f(fmaf(C[3], x, fmaf(C[4], s, C[5])));
    const float r = __builtin_amdgcn_rcpf(1.f + er);
    const float z = __builtin_amdgcn_rcpf(1.f + ez);
    const float q2 = fmaf(C[8], s, C[9]);
    const float ec = __builtin_amdgcn_exp2f(fmaf(r, q2, fmaf(C[6], x, C[7])));
    const float c = fmaf(-2.f, __builtin_amdgcn_rcpf(1.f + ec), 1.f);
    const float sc = s - c;
    const float zz = fmaf(-z, z, z);
    const float cc = fmaf(-c, c, 1.f);
    const float eta = fmaf(-z, cc, cc);               // (1 - z)(1 - c^2)
    const float rr = fmaf(-r, r, r);
    co[0] = eta * (q2 * (0.5f / LOG2E)) * rr;          // eta q r (1 - r)
    co[1] = sc * zz;                                   // (s - c) z (1 - z)
    co[2] = eta;
    co[3] = eta * r;
    J = fmaf(co[3], C[11], fmaf(co[1], C[10], fmaf(co[0], C[12] * (2.f * LOG2E), z)));
  } else if constexpr (CELL == C_TANH) {
    const float e = __builtin_amdgcn_exp2f(2.f * LOG2E * fmaf(C[0], x, fmaf(C[1], s, C[2])));
    const float f = fmaf(-2.f, __builtin_amdgcn_rcpf(1.f + e), 1.f);
    co[0] = fmaf(-f, f, 1.f);
    co[1] = co[2] = co[3] = 0.f;
    J = co[0] * C[1];
  } else {
    co[0] = 1.f;
    co[1] = co[2] = co[3] = 0.f;
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

// Wavefront totals of the last two computed tiles and the carries entering
// each of their wavefronts.
struct ScShared {
  float wA[2][SC_CW], wb[2][SC_CW];
  float cw[2][SC_CW];
  unsigned done[2];  // compute wavefronts finished with the tile in each buffer
  int stop;
  unsigned dmax[SC_CW];
  float red[SC_CW][12];
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

// The wavefront's total (wA, wb) into LDS buffer `buf`; the last compute
// wavefront to get here publishes the tile aggregate at once (tile 0 of a
// sequence only ever publishes its inclusive prefix).  Every compute
// wavefront executes the store; the others' offsets fall outside the
// resource.  LDS operations of a wavefront complete in order, so the totals
// written here are visible before its count is.
__device__ inline void sc_publish(const TimeArgs &a, int id, float wA, float wb, ScShared &sh, int buf) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, j = id / a.B;
  if (lane == 0) {
    sh.wA[buf][wid] = wA;
    sh.wb[buf][wid] = wb;
  }
  unsigned prev = 0;
  // the clobber keeps the compiler from moving memory accesses across
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
  const ScDesc d = sc_desc(a, id % a.B);
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
      if (++spins > PR_SPIN_LIMIT) {  // the fault is reported by the host; the carry poisons the rest
        if ((threadIdx.x & 63) == 0) spin_fault(st);
        return __builtin_nanf("");
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

// Look-back wavefront, for computed tile `id` whose wavefront totals are in
// LDS buffer `buf`: resolve its carry from the predecessors' descriptors,
// publish its inclusive prefix, and leave in LDS the carry entering each
// compute wavefront (lane w composes the totals of wavefronts 0 .. w - 1, once
// per tile rather than in every compute wavefront).  This wavefront issues no
// other memory operations, so its waits on the descriptors never queue behind
// the bulk loads and stores of the compute wavefronts.
__device__ inline void sc_lookback_tile(const TimeArgs &a, int id, ScShared &sh, int buf) {
  const int k = a.k, j = id / a.B, lane = threadIdx.x & 63;
  float totA = 1.f, totb = 0.f;
#pragma unroll
  for (int w = 0; w < SC_CW; w++) {
    totb = fmaf(sh.wA[buf][w], totb, sh.wb[buf][w]);
    totA *= sh.wA[buf][w];
  }
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
  w.x = __float_as_uint(fmaf(totA, carry, totb));
  w.y = tag_incl(k);
  __builtin_amdgcn_raw_buffer_store_b64(w, d.incl, lane == 0 ? (unsigned)j * 8u : SC_OOB, 0, SC_SC1);
  float pA = 1.f, pb = 0.f;
#pragma unroll
  for (int v = 0; v < SC_CW - 1; v++) {
    const float A = sh.wA[buf][v], b = sh.wb[buf][v];
    if (v < lane) {
      pb = fmaf(A, pb, b);
      pA *= A;
    }
  }
  if (lane < SC_CW) sh.cw[buf][lane] = fmaf(pA, carry, pb);
}

// Members common to the scalar-state policies.
struct ScBase {
  static constexpr int WPE = 4;  // wavefronts per SIMD the register budget is sized for
  using Args = TimeArgs;
  using Shared = ScShared;
  struct Consts {
    float c[SC_NC];
  };
  __device__ static void shared_init(Shared &sh) {
    sh.done[0] = 0;
    sh.done[1] = 0;
  }
  __device__ static void consts(const Args &a, Consts &K) {
#pragma unroll
    for (int i = 0; i < SC_NC; i++) K.c[i] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(a.coef[i])));
  }
  __host__ __device__ static int ntiles(const Args &a) { return a.ntiles; }
  __device__ static void lookback_tile(const Args &a, int id, Shared &sh, int buf) { sc_lookback_tile(a, id, sh, buf); }
};

// ---------------------------------------------------------------------------
// Newton sweep policy.  Scan positions are time steps; tile j, wavefront w,
// group q, lane l holds steps t0 + 4 (64 q + l) .. + 3 with t0 = j TILE +
// w WSTEPS.  Needs T % 4 == 0, so a lane's 4 steps are all inside or all
// outside [0, T).
// ---------------------------------------------------------------------------
template <int CELL, bool FIRST>
struct SweepPol : ScBase {
  // long tiles (3 groups per wavefront x 11 wavefronts, one block per CU):
  // few look-back stages per sequence, which the chain of carries pays for
  // one by one, with three wavefronts per SIMD to overlap memory and ALU
  static constexpr int WPE = 3;
  static constexpr int Q = 3, WSTEPS = Q * 64 * SC_V, TILE = SC_CW * WSTEPS;
  // raw inputs of one tile: x and the current iterate h per group, and the
  // state before the wavefront's first step (zero when its resource is empty)
  struct Raw {
    float4 x[Q], h[Q];
    float sw;
  };
  // a computed tile waiting for its carry
  struct Tile {
    float J[Q][SC_V], R[Q][SC_V], H[Q][SC_V];
    float iA[Q], ib[Q], tA[Q], tb[Q];
  };
  struct Lds {};
  struct Acc {
    unsigned dmax;
  };
  // the stop rule on the previous sweep's measure (every block exits once it holds)
  __device__ static bool open(const Args &a, Shared &sh) {
    return sweep_open(a.st, a.k, a.tol, a.T, a.max_iters, &sh.stop);
  }
  __device__ static bool full(const Args &a, int id) { return (id / a.B) * TILE + TILE <= a.T; }
  __device__ static void acc_init(Acc &c) { c.dmax = 0; }

  // In the first sweep the iterate is the zero guess and h is not read.
  // id < 0: no tile (empty resources: the loads return zeros and move no data)
  __device__ static void load(const TimeArgs &a, int id, Raw &R) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, k = a.k, B = a.B, T = a.T;
    const bool none = id < 0;
    id = none ? 0 : id;
    const int j = id / B, b = id % B;
    const int t0 = j * TILE + wid * WSTEPS;
    const unsigned rbytes = none ? 0u : (unsigned)T * 4u;
    const Rsrc rx = sc_rsrc(a.x + (size_t)b * T, rbytes);
    const Rsrc rh = sc_rsrc(a.h + (size_t)b * T, rbytes);
#pragma unroll
    for (int q = 0; q < Q; q++) {
      const unsigned off = toff(t0 + (q * 64 + lane) * SC_V, T);
      R.x[q] = ld4(rx, off);
      if (!FIRST) R.h[q] = ld4(rh, off);
    }
    // the state before step t0: h0 (t0 = 0), the predecessor tile's last
    // state from the previous sweep (wavefront 0), or h[t0 - 1], which this
    // block writes only after this load, later in this sweep
    const float *sb = a.x;
    unsigned nb = 0, so = 0;
    if (t0 == 0) {
      if (a.h0) { sb = a.h0 + b; nb = 4; }
    } else if (!FIRST && t0 < T) {
      if (wid == 0) { sb = a.bnd + (size_t)((k - 1) & 1) * a.ntiles + (b * a.tiles_per_seq + j - 1); nb = 4; }
      else { sb = a.h + (size_t)b * T; nb = (unsigned)T * 4u; so = (unsigned)(t0 - 1) * 4u; }
    }
    R.sw = ld1(sc_rsrc(sb, none ? 0u : nb), so);
  }

  // cell, Jacobian and residual of every step, lane-serial composition,
  // wavefront scans, totals and the aggregate
  template <bool FULL>
  __device__ static void compute(const TimeArgs &a, const Consts &K, int id, const Raw &R, Tile &Tl, ScShared &sh,
                                 Lds &, int buf) {
    const float *C = K.c;
    constexpr int V = SC_V;
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, T = a.T;
    const int t0 = (id / a.B) * TILE + wid * WSTEPS;
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
    sc_publish(a, id, wA, wb, sh, buf);
  }

  // update of the tile's steps from its carry, convergence measure, stores
  __device__ static void apply(const TimeArgs &a, const Consts &, int id, const Tile &Tl, const ScShared &sh, Lds &,
                               int buf, Acc &acc) {
    constexpr int V = SC_V;
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, k = a.k, B = a.B, T = a.T;
    const int j = id / B, b = id % B, L = b * a.tiles_per_seq + j;
    const int t0 = j * TILE + wid * WSTEPS;
    const bool full = j * TILE + TILE <= T;
    float c = sh.cw[buf][wid];  // dh entering this wavefront's steps
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
        acc.dmax = u > acc.dmax ? u : acc.dmax;
      }
      st4(rh, toff(t0 + (q * 64 + lane) * V, T), hn[0], hn[1], hn[2], hn[3]);
      if (q == Q - 1)  // the tile's last state, kept for the next sweep
        st1(rb, (full && wid == SC_CW - 1 && lane == 63) ? (unsigned)((k & 1) * a.ntiles + L) * 4u : SC_OOB, hn[V - 1]);
      c = fmaf(Tl.tA[q], c, Tl.tb[q]);
    }
  }

  // block maximum of |dh| into a shard of the sweep's convergence measure
  __device__ static void finish(const TimeArgs &a, Acc &acc, ScShared &sh) {
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const unsigned m = wave_max_dpp(acc.dmax);
    if (lane == 0 && wid < SC_CW) sh.dmax[wid] = m;
    __syncthreads();
    if (tid == 0) {
      unsigned v = sh.dmax[0];
      for (int w = 1; w < SC_CW; w++) v = sh.dmax[w] > v ? sh.dmax[w] : v;
      max_agent(&a.st->dslot[a.k & 3][blockIdx.x % PR_DSHARDS], v);
    }
  }
};

// ---------------------------------------------------------------------------
// Adjoint policy: lambda_t = g_t + J_{t+1} lambda_{t+1} (lambda_{T-1} =
// g_{T-1}) by a scan over reversed time, then per step the reverse-mode
// coefficients of the cell (recomputed from x and h, which the tile keeps)
// give dx_t, dh0 (t = 0) and the weight-gradient sums.  Scan position p
// holds step T - 1 - p; a lane's 4 steps are t_lo .. t_lo + 3 with t_lo =
// T - 4 - p0, visited from t_lo + 3 down.  Needs T % 4 == 0.
// ---------------------------------------------------------------------------
template <int CELL>
struct AdjPol : ScBase {
  static constexpr int WPE = 3;
  static constexpr int Q = 2, WSTEPS = Q * 64 * SC_V, TILE = SC_CW * WSTEPS;
  struct Raw {
    float4 x[Q], h[Q], g[Q];
    float hp;   // h before the wavefront's earliest step (0 at t = 0: h0 is taken then)
    float xn;   // x after the wavefront's latest step
    float h0b;  // h0 of the sequence (0 without h0)
  };
  struct Tile {
    float4 x[Q], h[Q];
    float hp, h0b;
    float iA[Q], ib[Q], tA[Q], tb[Q];
  };
  // per lane and group: the scan multipliers A_t = J_{t+1} and g_t of the
  // computed tile (lane-private slots, so no cross-wavefront hazard)
  struct Lds {
    float4 A[2][SC_CW][Q][64];
    float4 g[2][SC_CW][Q][64];
  };
  struct Acc {
    float v[10];
  };
  __device__ static bool open(const Args &, Shared &) {
    __syncthreads();
    return false;
  }
  __device__ static bool full(const Args &a, int id) { return (id / a.B) * TILE + TILE <= a.T; }
  __device__ static void acc_init(Acc &c) {
#pragma unroll
    for (int i = 0; i < 10; i++) c.v[i] = 0.f;
  }

  __device__ static int tlo(const TimeArgs &a, int id, int q) {
    const int wid = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int p0 = (id / a.B) * TILE + wid * WSTEPS + (q * 64 + lane) * SC_V;
    return a.T - SC_V - p0;
  }

  // id < 0: no tile (empty resources: the loads return zeros and move no data)
  __device__ static void load(const TimeArgs &a, int id, Raw &R) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, B = a.B, T = a.T;
    const bool none = id < 0;
    id = none ? 0 : id;
    const int b = id % B;
    const unsigned rbytes = none ? 0u : (unsigned)T * 4u;
    const Rsrc rx = sc_rsrc(a.x + (size_t)b * T, rbytes);
    const Rsrc rh = sc_rsrc(a.h + (size_t)b * T, rbytes);
    const Rsrc rg = sc_rsrc(a.g + (size_t)b * T, rbytes);
#pragma unroll
    for (int q = 0; q < Q; q++) {
      const int t = tlo(a, id, q);
      const unsigned off = (t >= 0 && t < T) ? (unsigned)t * 4u : SC_OOB;
      R.x[q] = ld4(rx, off);
      R.h[q] = ld4(rh, off);
      R.g[q] = ld4(rg, off);
    }
    // latest step of the wavefront: lane 0 of group 0; earliest: lane 63 of
    // the last group
    const int p_first = (id / B) * TILE + wid * WSTEPS;
    const int t_late = T - 1 - p_first, t_early = T - p_first - WSTEPS;
    (void)lane;
    R.xn = ld1(rx, toff(t_late + 1, T));
    R.hp = ld1(rh, toff(t_early - 1, T));
    R.h0b = ld1(sc_rsrc(a.h0 ? a.h0 + b : nullptr, none ? 0u : 4u), 0u);
  }

  template <bool FULL>
  __device__ static void compute(const TimeArgs &a, const Consts &K, int id, const Raw &R, Tile &Tl, ScShared &sh,
                                 Lds &lds, int buf) {
    const float *C = K.c;
    constexpr int V = SC_V;
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, T = a.T;
    // J of the step after the wavefront's latest step (lane 0, group 0)
    float Jn;
    {
      float f;
      scalar_cell<CELL>(C, R.h[0].w, R.xn, f, Jn);
    }
    float Jprev = 0.f;  // J at the earliest step of the previous group's lane 63
#pragma unroll
    for (int q = 0; q < Q; q++) {
      const int t = tlo(a, id, q);
      const bool in = FULL || t >= 0;
      const float xv[V] = {R.x[q].x, R.x[q].y, R.x[q].z, R.x[q].w};
      const float hv[V] = {R.h[q].x, R.h[q].y, R.h[q].z, R.h[q].w};
      // state before the lane's earliest step: the next lane's latest h
      const float last = q + 1 < Q ? rdlane(R.h[q + 1].w, 0) : R.hp;
      float s0 = shift_out(last, hv[V - 1]);
      if (t == 0) s0 = R.h0b;
      float J[V];
#pragma unroll
      for (int e = 0; e < V; e++) {
        float f;
        scalar_cell<CELL>(C, e == 0 ? s0 : hv[e - 1], xv[e], f, J[e]);
      }
      // A_e = J of step t + e + 1: own cells for e < 3, the previous lane's
      // earliest cell for e = 3 (zero after the sequence's last step)
      float A3 = shift_in(q == 0 ? Jn : Jprev, J[0]);
      if (t + V >= T) A3 = 0.f;
      Jprev = rdlane(J[0], 63);
      float Av[V] = {J[1], J[2], J[3], A3};
      float gv[V] = {R.g[q].x, R.g[q].y, R.g[q].z, R.g[q].w};
      if (!in) {
#pragma unroll
        for (int e = 0; e < V; e++) { Av[e] = 1.f; gv[e] = 0.f; }
      }
      float A = 1.f, bb = 0.f;
#pragma unroll
      for (int e = V - 1; e >= 0; e--) {
        bb = fmaf(Av[e], bb, gv[e]);
        A *= Av[e];
      }
      lds.A[buf][wid][q][lane] = make_float4(Av[0], Av[1], Av[2], Av[3]);
      lds.g[buf][wid][q][lane] = make_float4(gv[0], gv[1], gv[2], gv[3]);
      Tl.x[q] = R.x[q];
      Tl.h[q] = R.h[q];
      wave_scan_affine1(A, bb);
      Tl.iA[q] = A;
      Tl.ib[q] = bb;
      Tl.tA[q] = rdlane(A, 63);
      Tl.tb[q] = rdlane(bb, 63);
    }
    Tl.hp = R.hp;
    Tl.h0b = R.h0b;
    float wA = Tl.tA[0], wb = Tl.tb[0];
#pragma unroll
    for (int q = 1; q < Q; q++) {
      wb = fmaf(Tl.tA[q], wb, Tl.tb[q]);
      wA *= Tl.tA[q];
    }
    sc_publish(a, id, wA, wb, sh, buf);
  }

  __device__ static void apply(const TimeArgs &a, const Consts &K, int id, const Tile &Tl, const ScShared &sh,
                               Lds &lds, int buf, Acc &acc) {
    const float *C = K.c;
    constexpr int V = SC_V;
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, B = a.B, T = a.T;
    const int b = id % B;
    float c = sh.cw[buf][wid];  // lambda entering this wavefront (after its latest step)
    const Rsrc rl = sc_rsrc(a.lam ? a.lam + (size_t)b * T : nullptr, (unsigned)T * 4u);
    const Rsrc rd = sc_rsrc(a.dx ? a.dx + (size_t)b * T : nullptr, (unsigned)T * 4u);
    const Rsrc r0 = sc_rsrc(a.dh0 ? a.dh0 + b : nullptr, 4u);
#pragma unroll
    for (int q = 0; q < Q; q++) {
      const int t = tlo(a, id, q);
      const bool in = t >= 0;
      const float4 A4 = lds.A[buf][wid][q][lane], g4 = lds.g[buf][wid][q][lane];
      const float Av[V] = {A4.x, A4.y, A4.z, A4.w}, gv[V] = {g4.x, g4.y, g4.z, g4.w};
      const float xv[V] = {Tl.x[q].x, Tl.x[q].y, Tl.x[q].z, Tl.x[q].w};
      const float hv[V] = {Tl.h[q].x, Tl.h[q].y, Tl.h[q].z, Tl.h[q].w};
      const float last = q + 1 < Q ? rdlane(Tl.h[q + 1].w, 0) : Tl.hp;
      float s0 = shift_out(last, hv[V - 1]);
      if (t == 0) s0 = Tl.h0b;
      float lam = shift_in(c, fmaf(Tl.iA[q], c, Tl.ib[q]));
      float lv[V], dxv[V];
      float dh0 = 0.f;
#pragma unroll
      for (int e = V - 1; e >= 0; e--) {
        lam = fmaf(Av[e], lam, gv[e]);
        lv[e] = lam;
        const float s = e == 0 ? s0 : hv[e - 1];
        float co[4], J;
        scalar_vjp<CELL>(C, s, xv[e], co, J);
        const float l = in ? lam : 0.f;
        if constexpr (CELL == C_GRU) {
          const float ur = l * co[0], uz = l * co[1], un = l * co[2], an = l * co[3];
          dxv[e] = fmaf(C[15], un, fmaf(C[14], uz, C[13] * ur));
          acc.v[0] = fmaf(ur, xv[e], acc.v[0]);
          acc.v[1] = fmaf(uz, xv[e], acc.v[1]);
          acc.v[2] = fmaf(un, xv[e], acc.v[2]);
          acc.v[3] += ur;
          acc.v[4] += uz;
          acc.v[5] += un;
          acc.v[6] = fmaf(ur, s, acc.v[6]);
          acc.v[7] = fmaf(uz, s, acc.v[7]);
          acc.v[8] = fmaf(an, s, acc.v[8]);
          acc.v[9] += an;
        } else {
          const float u = l * co[0];
          dxv[e] = C[0] * u;
          acc.v[0] = fmaf(u, xv[e], acc.v[0]);
          acc.v[1] += u;
          acc.v[2] = fmaf(u, s, acc.v[2]);
        }
        if (e == 0) dh0 = J * l;
      }
      const unsigned off = (in && t < T) ? (unsigned)t * 4u : SC_OOB;
      st4_nt(rl, off, lv[0], lv[1], lv[2], lv[3]);
      st4_nt(rd, off, dxv[0], dxv[1], dxv[2], dxv[3]);
      st1(r0, t == 0 ? 0u : SC_OOB, dh0);
      c = fmaf(Tl.tA[q], c, Tl.tb[q]);
    }
  }

  // block sums of the weight-gradient partials, in the layout the reduction
  // kernel reads: [W_x (G), b_x (G), W_h (G), b_h (G)]
  __device__ static void finish(const TimeArgs &a, Acc &acc, ScShared &sh) {
    constexpr int G = CELL == C_GRU ? 3 : 1, P = 4 * G;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    float v[P];
    if constexpr (CELL == C_GRU) {
      const float m[12] = {acc.v[0], acc.v[1], acc.v[2], acc.v[3], acc.v[4], acc.v[5],
                           acc.v[6], acc.v[7], acc.v[8], acc.v[3], acc.v[4], acc.v[9]};
#pragma unroll
      for (int i = 0; i < 12; i++) v[i] = m[i];
    } else {
      v[0] = acc.v[0]; v[1] = acc.v[1]; v[2] = acc.v[2]; v[3] = acc.v[1];
    }
#pragma unroll
    for (int i = 0; i < P; i++) {
      const float w = wave_total(v[i]);
      if (lane == 0 && wid < SC_CW) sh.red[wid][i] = w;
    }
    __syncthreads();
    if (tid < P) {
      float s = 0.f;
      for (int w = 0; w < SC_CW; w++) s += sh.red[w][tid];
      a.part[(size_t)blockIdx.x * P + tid] = s;
    }
  }
};

int scalar_tile() { return SweepPol<C_GRU, false>::TILE; }
int scalar_adj_tile() { return AdjPol<C_GRU>::TILE; }

hipError_t launch_zero_coef(void *p, size_t bytes, const float *Wx, const float *bx, const float *Wh,
                            const float *bh, int cell, float *coef, hipStream_t s) {
  const size_t n16 = bytes / 16, ntail = bytes % 16;
  size_t blocks = (n16 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks == 0) blocks = 1;
  hipLaunchKernelGGL(k_zero_coef, dim3((unsigned)blocks), dim3(256), 0, s, (uint4 *)p, n16,
                     (unsigned char *)p + n16 * 16, ntail, Wx, bx, Wh, bh, cell, coef);
  return hipGetLastError();
}

template <int CELL>
static hipError_t scalar_sweep_cell(const TimeArgs &a, hipStream_t s) {
  return a.k == 1 ? pipe_launch<SweepPol<CELL, true>>(a, s) : pipe_launch<SweepPol<CELL, false>>(a, s);
}

hipError_t launch_scalar_sweep(int cell, const TimeArgs &a, hipStream_t s) {
  switch (cell) {
    case C_GRU: return scalar_sweep_cell<C_GRU>(a, s);
    case C_TANH: return scalar_sweep_cell<C_TANH>(a, s);
    case C_LINEAR: return scalar_sweep_cell<C_LINEAR>(a, s);
    default: return hipErrorInvalidValue;
  }
}

// The adjoint writes one row of weight-gradient partials per block (the
// block count is returned in a.nparts for the reduction).
hipError_t launch_scalar_adjoint(int cell, TimeArgs &a, hipStream_t s) {
  int grid = 0;
  hipError_t e;
  switch (cell) {
    case C_GRU: e = pipe_launch<AdjPol<C_GRU>>(a, s, &grid); break;
    case C_TANH: e = pipe_launch<AdjPol<C_TANH>>(a, s, &grid); break;
    case C_LINEAR: e = pipe_launch<AdjPol<C_LINEAR>>(a, s, &grid); break;
    default: return hipErrorInvalidValue;
  }
  a.nparts = grid;
  return e;
}

}  // namespace pr

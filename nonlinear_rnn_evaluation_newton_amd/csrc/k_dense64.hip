// Full-DEER path for a dense 64 x 64 Jacobian (GRU, n = 64): the cubic-cost
// case the DEER summary flags ("Surprising findings": the explicit Jacobian
// and its matrix products scale as O(n^3)), on fp32 MFMA.
//
// A sweep is four launches:
//  1. gates: a = W_h h_{t-1} for all steps on MFMA, then per step the GRU
//     gates and the vectors that define J_t = diag(z) + diag(alpha) W_hz +
//     diag(beta) W_hn + diag(gamma) W_hr, plus the residual r_t = f_t - h_t.
//     J_t itself (16 KB per step) is never stored: it is rebuilt on the fly.
//  2. chunk products: each wavefront composes the affine operators of L = 64
//     consecutive steps, P = J_L ... J_1 on MFMA (v_mfma_f32_32x32x2_f32) and
//     the offset b by a matrix-vector chain, and stores (P, b).
//  3. chunk carries: per sequence, c_{j+1} = P_j c_j + b_j.
//  4. chunk replay: each chunk re-runs dh_t = J_t dh_{t-1} + r_t from its
//     carry, updates h in place and measures max |dh|.
// The adjoint runs the same scan backwards in time with J^T (step 2 with the
// Jacobian transposed, step 4 as lambda_t = J_{t+1}^T lambda_{t+1} + g_t).
//
// Register trick of step 2: a 32x32 MFMA result lane holds rows
// 8(r/4) + 4(l/32) + r%4 of column l%32 in register r.  Taking the k index of
// the next product in that same order makes register r of the previous
// product exactly the B operand of k-step r, so the running product never
// leaves the accumulators; only the A operand (J_t) is rebuilt, one value per
// lane and k-step, from the three weight matrices held in LDS.
#include "internal.h"

namespace pr {

typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_d;

constexpr int WLD = 68;  // padded LDS row stride (floats) of 64-wide matrices

__device__ inline int r0_of(int r) { return 8 * (r >> 2) + (r & 3); }

// W_h [192][64] into LDS (stride WLD)
__device__ inline void d64_stage(const D64Args &a, float *sW) {
  for (int e = threadIdx.x; e < 192 * 16; e += 256) {
    const int row = e >> 4, c4 = (e & 15) * 4;
    *reinterpret_cast<float4 *>(&sW[row * WLD + c4]) = *reinterpret_cast<const float4 *>(a.Wh + row * 64 + c4);
  }
}

// ---------------------------------------------------------------------------
// 1. gates: per step the GRU gates on top of W_h h_{t-1} (MFMA).  Outputs:
//    GM_SWEEP  [row][5][64]: z, alpha, beta, gamma, res (J_t = diag(z) +
//              diag(alpha) W_hz + diag(beta) W_hn + diag(gamma) W_hr)
//    GM_ADJ    the same with eta = (1 - z)(1 - c^2) in place of res
//    GM_QUASI  [row][2][64]: the Jacobian's diagonal (or 0) and res, plus
//              each chunk's per-channel aggregate (see the quasi sweep below)
// ---------------------------------------------------------------------------
enum { GM_SWEEP = 0, GM_ADJ = 1, GM_QUASI = 2 };

// Persistent over units of D64_L steps of one sequence (unit = chunk):
// W_h stays in LDS; each block prefetches the states entering its next
// unit's rows (the MFMA's input) while it computes the current one, and
// issues the current unit's U and iterate loads before its MFMA, which
// covers their latency.  MFMA layout: wavefront w computes rows
// [32 (w & 1), +32) x channels [32 (w >> 1), +32) of all three gates, so a
// lane ends up holding, for one channel, the three pre-activations of 16
// rows, and the gate arithmetic runs in registers with no transpose.
template <int MODE>
__global__ __launch_bounds__(256) void k_d64_gates(const D64Args a) {
  __shared__ int s_stop;
  __shared__ __attribute__((aligned(16))) float sW[192 * WLD];
  __shared__ __attribute__((aligned(16))) float sH[64 * WLD];
  __shared__ float sAgg[2][2][64];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  if (MODE != GM_ADJ && sweep_open(a.st, a.k, a.tol, a.T, a.max_iters, &s_stop)) return;
  const int T = a.T, cps = a.cps, nunits = a.nchunks, G = gridDim.x;
  const bool first = MODE != GM_ADJ && a.k == 1;  // the iterate is h = 0 before sweep 1
  const int rb = wid & 1, cbk = wid >> 1, hl = lane >> 5, li = lane & 31;
  const int c = cbk * 32 + li;  // this lane's channel
  const float bhr = a.bh ? a.bh[c] : 0.f, bhz = a.bh ? a.bh[64 + c] : 0.f, bhn = a.bh ? a.bh[128 + c] : 0.f;
  float wr = 0.f, wz = 0.f, wn = 0.f;
  if (MODE == GM_QUASI) {
    wr = a.Wh[c * 64 + c];
    wz = a.Wh[(64 + c) * 64 + c];
    wn = a.Wh[(128 + c) * 64 + c];
  }
  const bool diag = a.approx == APX_DIAG;

  // row of MFMA result register r within the unit
  auto row_of = [&](int r) { return 32 * rb + 8 * (r >> 2) + 4 * hl + (r & 3); };
  // This thread's share of the states entering a unit's 64 rows (h_{t-1},
  // h0 at t = 0, or 0; bit m of zmask set when share m must be 0).
  // Addresses are clamped into the unit, so the loads are unconditional.
  auto load_states = [&](int unit, float4 (&hs)[4], unsigned &zmask) __attribute__((always_inline)) {
    const int b = unit / cps, t0 = (unit % cps) * D64_L, nr = min(D64_L, T - t0);
    const size_t row0 = (size_t)b * T + t0;
    zmask = 0;
#pragma unroll
    for (int m = 0; m < 4; m++) {
      const int e = tid + 256 * m, rr = e >> 4, c4 = (e & 15) * 4;
      const int rc = min(rr, nr - 1), t = t0 + rc;
      const float *src = t > 0 ? a.h + (row0 + rc - 1) * 64 + c4 : (a.h0 ? a.h0 + (size_t)b * 64 + c4 : a.h + row0 * 64 + c4);
      hs[m] = *reinterpret_cast<const float4 *>(src);
      const bool zero = rr >= nr || (t > 0 ? first : a.h0 == nullptr);
      zmask |= zero ? 1u << m : 0u;
    }
  };

  int unit = blockIdx.x;
  if (unit >= nunits) return;
  float4 nhs[4];
  unsigned nz;
  load_states(unit, nhs, nz);
  d64_stage(a, sW);
  while (true) {
    __syncthreads();  // the previous unit's MFMA has read sH (and W_h is staged)
#pragma unroll
    for (int m = 0; m < 4; m++) {
      const int e = tid + 256 * m, rr = e >> 4, c4 = (e & 15) * 4;
      const float4 z4 = make_float4(0.f, 0.f, 0.f, 0.f);
      *reinterpret_cast<float4 *>(&sH[rr * WLD + c4]) = ((nz >> m) & 1u) ? z4 : nhs[m];
    }
    __syncthreads();
    const int b = unit / cps, j = unit % cps, t0 = j * D64_L, nr = min(D64_L, T - t0);
    const size_t row0 = (size_t)b * T + t0;
    // U and the iterate at this lane's 16 rows (rows past the end load the
    // last row and are not stored), then the next unit's states
    float u[3][16], hc[16];
#pragma unroll
    for (int r = 0; r < 16; r++) {
      const size_t row = row0 + min(row_of(r), nr - 1);
#pragma unroll
      for (int g = 0; g < 3; g++) u[g][r] = a.U[row * 192 + 64 * g + c];
      hc[r] = MODE == GM_ADJ ? 0.f : a.h[row * 64 + c];
    }
    const int next = unit + G;
    load_states(next < nunits ? next : unit, nhs, nz);  // the last unit reloads itself

    f32x16_d acc[3];
#pragma unroll
    for (int g = 0; g < 3; g++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[g][r] = 0.f;
#pragma unroll 4
    for (int s = 0; s < 32; s++) {
      const int kk = 2 * s + hl;
      const float av = sH[(32 * rb + li) * WLD + kk];
#pragma unroll
      for (int g = 0; g < 3; g++)
        acc[g] = __builtin_amdgcn_mfma_f32_32x32x2f32(av, sW[(64 * g + 32 * cbk + li) * WLD + kk], acc[g], 0, 0, 0);
    }

    float ga[4], gb[4];  // quasi: aggregates of this lane's four runs of 4 rows
#pragma unroll
    for (int r4 = 0; r4 < 4; r4++) {
      ga[r4] = 1.f;
      gb[r4] = 0.f;
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const int r = 4 * r4 + q, R = row_of(r);
        const bool live = R < nr;
        const size_t row = row0 + R;
        const float sv = sH[R * WLD + c];
        const float ar = acc[0][r] + u[0][r] + bhr;
        const float az = acc[1][r] + u[1][r] + bhz;
        const float qv = acc[2][r] + bhn;
        const float rg = fsigm(ar), z = fsigm(az);
        const float cc = ftanh(fmaf(rg, qv, u[2][r]));
        const float eta = (1.f - z) * (1.f - cc * cc);
        if constexpr (MODE == GM_QUASI) {
          const float f = fmaf(z, sv - cc, cc);
          const float Jd = diag ? z + (sv - cc) * z * (1.f - z) * wz + eta * rg * (wn + qv * (1.f - rg) * wr) : 0.f;
          const float res = f - (first ? 0.f : hc[r]);
          if (live) {
            a.gates[row * 128 + c] = Jd;
            a.gates[row * 128 + 64 + c] = res;
          }
          gb[r4] = live ? fmaf(Jd, gb[r4], res) : gb[r4];
          ga[r4] = live ? Jd * ga[r4] : ga[r4];
        } else if (live) {
          float *Gr = a.gates + row * 320;
          Gr[c] = z;
          Gr[64 + c] = (sv - cc) * z * (1.f - z);
          Gr[128 + c] = eta * rg;
          Gr[192 + c] = eta * qv * rg * (1.f - rg);
          Gr[256 + c] = MODE == GM_ADJ ? eta : fmaf(z, sv - cc, cc) - (first ? 0.f : hc[r]);
        }
      }
    }
    if constexpr (MODE == GM_QUASI) {
      // rows 8 r4 + [0, 4) sit in the lower half-wave, 8 r4 + [4, 8) in the
      // upper one: compose each pair in time order, then the four runs
      float A = 1.f, B = 0.f;
#pragma unroll
      for (int r4 = 0; r4 < 4; r4++) {
        const float pa = __shfl_xor(ga[r4], 32, 64), pb = __shfl_xor(gb[r4], 32, 64);
        const float ea = hl ? pa : ga[r4], eb = hl ? pb : gb[r4];  // earlier 4 rows
        const float la = hl ? ga[r4] : pa, lb = hl ? gb[r4] : pb;  // later 4 rows
        const float a8 = la * ea, b8 = fmaf(la, eb, lb);
        B = fmaf(a8, B, b8);
        A *= a8;
      }
      if (hl == 0) {
        sAgg[rb][0][c] = A;
        sAgg[rb][1][c] = B;
      }
      __syncthreads();
      if (tid < 64) {
        const float a0 = sAgg[0][0][tid], b0 = sAgg[0][1][tid], a1 = sAgg[1][0][tid], b1 = sAgg[1][1][tid];
        const size_t o = ((size_t)b * 64 + tid) * cps + j;
        a.aggP[o] = a1 * a0;
        a.aggb[o] = fmaf(a1, b0, b1);
      }
    }
    if (next >= nunits) break;
    unit = next;
  }
}

// ---------------------------------------------------------------------------
// 2. chunk products on MFMA
// ---------------------------------------------------------------------------
// Weight matrices in LDS, laid out so that lane (row i, k-run) reads 4
// consecutive k with one 16-byte load: forward W*[i][k]; transposed
// (adjoint) W*[k][i].  Order: z, n, r (the coefficients alpha, beta, gamma).
template <bool TR>
__device__ inline void stage_w3(const float *Wh, float *sW) {
  const int mats[3] = {64, 128, 0};  // row offsets of W_hz, W_hn, W_hr in W_h [192, 64]
  for (int e = threadIdx.x; e < 3 * 64 * 64; e += blockDim.x) {
    const int m = e / 4096, rem = e % 4096, i = rem / 64, k = rem % 64;
    const float v = TR ? Wh[(mats[m] + k) * 64 + i] : Wh[(mats[m] + i) * 64 + k];
    sW[m * 64 * WLD + i * WLD + k] = v;
  }
}

template <bool ADJ>
__global__ __launch_bounds__(256) void k_d64_scanA(const D64Args a) {
  __shared__ int s_stop;
  __shared__ __attribute__((aligned(16))) float sW[3 * 64 * WLD];
  __shared__ __attribute__((aligned(16))) float sB[4][64];
  // per wavefront, two steps' coefficients: z, alpha, beta, gamma, right-hand side
  __shared__ __attribute__((aligned(16))) float sCo[4][2][5][64];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  if (!ADJ && sweep_is_stopped(a.st, &s_stop)) return;
  stage_w3<ADJ>(a.Wh, sW);
  __syncthreads();
  const int chunk = blockIdx.x * 4 + wid;
  if (chunk >= a.nchunks) return;
  const int b = chunk / a.cps, j = chunk % a.cps, T = a.T;
  const int h = lane >> 5, li = lane & 31;
  const float *sWz = sW, *sWn = sW + 64 * WLD, *sWr = sW + 2 * 64 * WLD;

  f32x16_d P[2][2];  // running product, [row block][column block]
#pragma unroll
  for (int ob = 0; ob < 2; ob++)
#pragma unroll
    for (int cb = 0; cb < 2; cb++)
#pragma unroll
      for (int r = 0; r < 16; r++) P[ob][cb][r] = (ob == cb && r0_of(r) + 4 * h == li) ? 1.f : 0.f;
  float bk[2][16];  // offset at this lane's k set {ib*32 + r0(r) + 4h}
  float brow[2];    // offset at this lane's rows {ob*32 + li}
#pragma unroll
  for (int ib = 0; ib < 2; ib++)
#pragma unroll
    for (int r = 0; r < 16; r++) bk[ib][r] = 0.f;
  brow[0] = brow[1] = 0.f;

  // Entry `lane` of one step's coefficients (z, alpha, beta, gamma of the
  // row holding the Jacobian, the right-hand side of the step's own row),
  // fetched a step ahead; addresses are clamped into the sequence and the
  // adjoint's last step (J = 0) or a step past the chunk read as zero.
  auto fetch = [&](int sidx, float (&co)[5]) __attribute__((always_inline)) {
    const int sc = min(sidx, T - 1);
    const int t = ADJ ? T - 1 - sc : sc;
    const int cr = ADJ ? t + 1 : t;  // row holding the Jacobian's coefficients
    const bool live = cr < T && sidx < T;
    const size_t rowc = (size_t)b * T + (cr < T ? cr : t), rowt = (size_t)b * T + t;
#pragma unroll
    for (int m = 0; m < 4; m++) co[m] = a.gates[rowc * 320 + 64 * m + lane];
    co[4] = ADJ ? a.g[rowt * 64 + lane] : a.gates[rowt * 320 + 256 + lane];
#pragma unroll
    for (int m = 0; m < 4; m++) co[m] = live ? co[m] : 0.f;
  };
  float co[5];
  fetch(j * D64_L, co);

  for (int s = 0; s < D64_L; s++) {
    const int sidx = j * D64_L + s;  // position in scan order
    if (sidx >= T) break;
    float(*cs)[64] = sCo[wid][s & 1];
#pragma unroll
    for (int m = 0; m < 5; m++) cs[m][lane] = co[m];
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // LDS order within the wavefront
    __builtin_amdgcn_wave_barrier();
    fetch(sidx + 1, co);  // the next step's, in flight during this step's products
    float zk[2][16];  // z at this lane's rows of P (same index pattern as the k set)
#pragma unroll
    for (int ib = 0; ib < 2; ib++)
#pragma unroll
      for (int r4 = 0; r4 < 4; r4++) {
        const int kb = ib * 32 + 8 * r4 + 4 * h;
        const float4 zv = *reinterpret_cast<const float4 *>(&cs[0][kb]);
        zk[ib][4 * r4 + 0] = zv.x; zk[ib][4 * r4 + 1] = zv.y; zk[ib][4 * r4 + 2] = zv.z; zk[ib][4 * r4 + 3] = zv.w;
      }
    float crow[3][2], zrow[2], brhs[2];
#pragma unroll
    for (int ob = 0; ob < 2; ob++) {
      const int i = ob * 32 + li;
      zrow[ob] = cs[0][i];
#pragma unroll
      for (int m = 0; m < 3; m++) crow[m][ob] = cs[m + 1][i];
      brhs[ob] = cs[4][i];
    }
    // P_new = diag(z) P + M P,  b_new = z * b + M b + rhs
    f32x16_d Pn[2][2];
#pragma unroll
    for (int ob = 0; ob < 2; ob++)
#pragma unroll
      for (int cb = 0; cb < 2; cb++)
#pragma unroll
        for (int r = 0; r < 16; r++) Pn[ob][cb][r] = zk[ob][r] * P[ob][cb][r];
    float part[2] = {0.f, 0.f};
#pragma unroll
    for (int ib = 0; ib < 2; ib++) {
#pragma unroll
      for (int r4 = 0; r4 < 4; r4++) {
        const int kb = ib * 32 + 8 * r4 + 4 * h;
        float ck[3][4];  // adjoint: coefficients at this run of k
        if (ADJ) {
#pragma unroll
          for (int m = 0; m < 3; m++) {
            const float4 cv = *reinterpret_cast<const float4 *>(&cs[m + 1][kb]);
            ck[m][0] = cv.x; ck[m][1] = cv.y; ck[m][2] = cv.z; ck[m][3] = cv.w;
          }
        }
#pragma unroll
        for (int ob = 0; ob < 2; ob++) {
          const int i = ob * 32 + li;
          const float4 wz = *reinterpret_cast<const float4 *>(&sWz[i * WLD + kb]);
          const float4 wn = *reinterpret_cast<const float4 *>(&sWn[i * WLD + kb]);
          const float4 wr = *reinterpret_cast<const float4 *>(&sWr[i * WLD + kb]);
          const float wzv[4] = {wz.x, wz.y, wz.z, wz.w}, wnv[4] = {wn.x, wn.y, wn.z, wn.w},
                      wrv[4] = {wr.x, wr.y, wr.z, wr.w};
#pragma unroll
          for (int q = 0; q < 4; q++) {
            const int r = 4 * r4 + q;
            float jv;
            if (ADJ) jv = fmaf(ck[0][q], wzv[q], fmaf(ck[1][q], wnv[q], ck[2][q] * wrv[q]));
            else jv = fmaf(crow[0][ob], wzv[q], fmaf(crow[1][ob], wnv[q], crow[2][ob] * wrv[q]));
#pragma unroll
            for (int cb = 0; cb < 2; cb++)
              Pn[ob][cb] = __builtin_amdgcn_mfma_f32_32x32x2f32(jv, P[ib][cb][r], Pn[ob][cb], 0, 0, 0);
            part[ob] = fmaf(jv, bk[ib][r], part[ob]);
          }
        }
      }
    }
#pragma unroll
    for (int ob = 0; ob < 2; ob++) {
      part[ob] += __shfl_xor(part[ob], 32, 64);
      brow[ob] = fmaf(zrow[ob], brow[ob], part[ob] + brhs[ob]);
    }
    // redistribute b to the k layout through this wavefront's LDS row
    if (lane < 32) {
      sB[wid][lane] = brow[0];
      sB[wid][32 + lane] = brow[1];
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int ib = 0; ib < 2; ib++)
#pragma unroll
      for (int r4 = 0; r4 < 4; r4++) {
        const float4 v = *reinterpret_cast<const float4 *>(&sB[wid][ib * 32 + 8 * r4 + 4 * h]);
        bk[ib][4 * r4 + 0] = v.x; bk[ib][4 * r4 + 1] = v.y; bk[ib][4 * r4 + 2] = v.z; bk[ib][4 * r4 + 3] = v.w;
      }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int ob = 0; ob < 2; ob++)
#pragma unroll
      for (int cb = 0; cb < 2; cb++) P[ob][cb] = Pn[ob][cb];
  }
  float *Po = a.aggP + (size_t)chunk * 4096;
#pragma unroll
  for (int ob = 0; ob < 2; ob++)
#pragma unroll
    for (int cb = 0; cb < 2; cb++)
#pragma unroll
      for (int r = 0; r < 16; r++) Po[(ob * 32 + r0_of(r) + 4 * h) * 64 + cb * 32 + li] = P[ob][cb][r];
  if (lane < 32) {
    a.aggb[(size_t)chunk * 64 + lane] = brow[0];
    a.aggb[(size_t)chunk * 64 + 32 + lane] = brow[1];
  }
}

// ---------------------------------------------------------------------------
// 3. chunk carries, one block per sequence
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_d64_scanB(const D64Args a) {
  __shared__ int s_stop;
  __shared__ float sc[64];
  if (!a.adjoint && sweep_is_stopped(a.st, &s_stop)) return;
  const int tid = threadIdx.x, b = blockIdx.x;
  const int i = tid >> 2, q = tid & 3;
  if (tid < 64) sc[tid] = 0.f;
  __syncthreads();
  constexpr int PF = 8;  // chunks prefetched ahead of the carry chain (matrix rows and offsets)
  float4 pv[PF][4];
  float bv[PF];
  const int c0 = b * a.cps;
  auto loadP = [&](int slot, int chunk) {
    const float *P = a.aggP + (size_t)chunk * 4096 + i * 64 + q * 16;
#pragma unroll
    for (int m = 0; m < 4; m++) pv[slot][m] = *reinterpret_cast<const float4 *>(P + 4 * m);
    bv[slot] = a.aggb[(size_t)chunk * 64 + i];
  };
  // ring slots are static (the loop is unrolled by PF) and the loads are
  // unconditional (chunk indices clamped), so no wait drains the ring early
#pragma unroll
  for (int f = 0; f < PF; f++) loadP(f, c0 + min(f, a.cps - 1));
  for (int j0 = 0; j0 < a.cps; j0 += PF) {
#pragma unroll
    for (int f = 0; f < PF; f++) {
      const int j = j0 + f;
      if (j >= a.cps) break;
      const int chunk = c0 + j;
      const float4 cur[4] = {pv[f][0], pv[f][1], pv[f][2], pv[f][3]};
      const float bj = q == 0 ? bv[f] : 0.f;
      loadP(f, c0 + min(j + PF, a.cps - 1));
      float s = 0.f;
#pragma unroll
      for (int m = 0; m < 4; m++) {
        const int k = q * 16 + 4 * m;
        s = fmaf(cur[m].x, sc[k], s);
        s = fmaf(cur[m].y, sc[k + 1], s);
        s = fmaf(cur[m].z, sc[k + 2], s);
        s = fmaf(cur[m].w, sc[k + 3], s);
      }
      s += __shfl_xor(s, 1, 64);
      s += __shfl_xor(s, 2, 64);
      if (tid < 64) a.carry[(size_t)chunk * 64 + tid] = sc[tid];
      lds_barrier();  // (keeps the prefetched chunks in flight)
      if (q == 0) sc[i] = s + bj;
      lds_barrier();
    }
  }
}

// ---------------------------------------------------------------------------
// 4. chunk replay (one wavefront per chunk, lane = state row)
// ---------------------------------------------------------------------------
template <bool ADJ>
__global__ __launch_bounds__(256) void k_d64_scanC(const D64Args a) {
  __shared__ int s_stop;
  __shared__ __attribute__((aligned(16))) float sY[4][3][64];
  __shared__ unsigned s_dmax[4];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  if (!ADJ && sweep_is_stopped(a.st, &s_stop)) return;
  const int chunk = blockIdx.x * 4 + wid;
  unsigned dmax = 0;
  if (chunk < a.nchunks) {
    const int b = chunk / a.cps, j = chunk % a.cps, T = a.T;
    const int i = lane;
    // this lane's weights: forward row i of W_hz, W_hn, W_hr; adjoint column i
    float w[3][64];
    const int mats[3] = {64, 128, 0};
#pragma unroll
    for (int m = 0; m < 3; m++)
#pragma unroll
      for (int k = 0; k < 64; k++) w[m][k] = ADJ ? a.Wh[(mats[m] + k) * 64 + i] : a.Wh[(mats[m] + i) * 64 + k];
    float y = a.carry[(size_t)chunk * 64 + i];
    const bool first = !ADJ && a.k == 1;
    // this lane's per-step values, fetched a step ahead (rows clamped into
    // the sequence): forward z, alpha, beta, gamma, res and the iterate at
    // row t; adjoint z, alpha, beta, gamma at row t + 1 (0 past the end) and g
    auto fetch = [&](int sidx, float (&co)[6]) __attribute__((always_inline)) {
      const int t = ADJ ? T - 1 - min(sidx, T - 1) : min(sidx, T - 1);
      const size_t row = (size_t)b * T + t;
      if (!ADJ) {
#pragma unroll
        for (int m = 0; m < 5; m++) co[m] = a.gates[row * 320 + 64 * m + i];
        co[5] = a.h[row * 64 + i];
      } else {
        const bool live = t + 1 < T;
        const size_t rc = live ? row + 1 : row;
#pragma unroll
        for (int m = 0; m < 4; m++) co[m] = a.gates[rc * 320 + 64 * m + i];
#pragma unroll
        for (int m = 0; m < 4; m++) co[m] = live ? co[m] : 0.f;
        co[4] = a.g[row * 64 + i];
        co[5] = 0.f;
      }
    };
    float cn[6];
    fetch(j * D64_L, cn);
    for (int s = 0; s < D64_L; s++) {
      const int sidx = j * D64_L + s;
      if (sidx >= T) break;
      const int t = ADJ ? T - 1 - sidx : sidx;
      const size_t row = (size_t)b * T + t;
      float co[6];
#pragma unroll
      for (int m = 0; m < 6; m++) co[m] = cn[m];
      fetch(sidx + 1, cn);
      float yn;
      if (!ADJ) {
        sY[wid][0][i] = y;
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // LDS order within the wavefront
        __builtin_amdgcn_wave_barrier();
        float sz = 0.f, sn = 0.f, sr = 0.f;
#pragma unroll
        for (int k4 = 0; k4 < 16; k4++) {
          const float4 v = *reinterpret_cast<const float4 *>(&sY[wid][0][4 * k4]);
          const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int q = 0; q < 4; q++) {
            sz = fmaf(w[0][4 * k4 + q], vv[q], sz);
            sn = fmaf(w[1][4 * k4 + q], vv[q], sn);
            sr = fmaf(w[2][4 * k4 + q], vv[q], sr);
          }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_wave_barrier();
        yn = fmaf(co[0], y, fmaf(co[1], sz, fmaf(co[2], sn, fmaf(co[3], sr, co[4]))));
        a.h[row * 64 + i] = (first ? 0.f : co[5]) + yn;
        const unsigned u = __float_as_uint(fabsf(yn));
        dmax = u > dmax ? u : dmax;
      } else {
        sY[wid][0][i] = co[1] * y;
        sY[wid][1][i] = co[2] * y;
        sY[wid][2][i] = co[3] * y;
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_wave_barrier();
        float acc = 0.f;
#pragma unroll
        for (int m = 0; m < 3; m++)
#pragma unroll
          for (int k4 = 0; k4 < 16; k4++) {
            const float4 v = *reinterpret_cast<const float4 *>(&sY[wid][m][4 * k4]);
            acc = fmaf(w[m][4 * k4], v.x, acc);
            acc = fmaf(w[m][4 * k4 + 1], v.y, acc);
            acc = fmaf(w[m][4 * k4 + 2], v.z, acc);
            acc = fmaf(w[m][4 * k4 + 3], v.w, acc);
          }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_wave_barrier();
        yn = fmaf(co[0], y, acc) + co[4];
        a.lam[row * 64 + i] = yn;
      }
      y = yn;
    }
  }
  if (!ADJ) {
    dmax = wave_max_u32(dmax);
    if (lane == 0) s_dmax[wid] = dmax;
    __syncthreads();
    if (tid == 0) {
      unsigned m = s_dmax[0];
      for (int q = 1; q < 4; q++) m = s_dmax[q] > m ? s_dmax[q] : m;
      max_agent(&a.st->dslot[a.k & 3][blockIdx.x % PR_DSHARDS], m);
    }
  }
}

// ---------------------------------------------------------------------------
// adjoint epilogue: gate pre-activation gradients and the shifted states
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_d64_adj_epi(const D64AdjArgs a) {
  const size_t e = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t rows = (size_t)a.B * a.T;
  if (e >= rows * 64) return;
  const size_t row = e >> 6;
  const int i = (int)(e & 63);
  const int t = (int)(row % a.T), b = (int)(row / a.T);
  const float l = a.lam[e];
  const float *G = a.gates + row * 320;
  const float al = G[64 + i], be = G[128 + i], ga = G[192 + i], eta = G[256 + i];
  a.dU[row * 192 + i] = l * ga;        // r gate
  a.dU[row * 192 + 64 + i] = l * al;   // z gate
  a.dU[row * 192 + 128 + i] = l * eta; // n gate (input part)
  a.dA[row * 192 + i] = l * ga;
  a.dA[row * 192 + 64 + i] = l * al;
  a.dA[row * 192 + 128 + i] = l * be;  // n gate (recurrent part, inside r * (.))
  a.hprev[e] = t > 0 ? a.h[e - 64] : (a.h0 ? a.h0[(size_t)b * 64 + i] : 0.f);
}

// dh0 = J_0^T lambda_0, with J_0 from the gates of step 0
__global__ __launch_bounds__(64) void k_d64_dh0(const D64AdjArgs a) {
  const int b = blockIdx.x, i = threadIdx.x;
  const size_t row = (size_t)b * a.T;
  const float *G = a.gates + row * 320;
  const float *L = a.lam + row * 64;
  float acc = G[i] * L[i];
  for (int k = 0; k < 64; k++) {
    const float lk = L[k];
    acc = fmaf(G[64 + k] * lk, a.Wh[(64 + k) * 64 + i], acc);
    acc = fmaf(G[128 + k] * lk, a.Wh[(128 + k) * 64 + i], acc);
    acc = fmaf(G[192 + k] * lk, a.Wh[k * 64 + i], acc);
  }
  a.dh0[(size_t)b * 64 + i] = acc;
}

// Column sums in fp64 in a fixed order: block q sums rows [q*R, (q+1)*R) of
// every column (coalesced across threads), then one pass sums the blocks.
constexpr int CS_BLOCKS = 512;
__global__ __launch_bounds__(256) void k_colsum_part(const float *X, int rows, int cols, double *part) {
  const int R = (rows + CS_BLOCKS - 1) / CS_BLOCKS;
  const int r0 = blockIdx.x * R, r1 = min(rows, r0 + R);
  for (int c = threadIdx.x; c < cols; c += 256) {
    double acc = 0.0;
    for (int r = r0; r < r1; r++) acc += (double)X[(size_t)r * cols + c];
    part[(size_t)blockIdx.x * cols + c] = acc;
  }
}
__global__ __launch_bounds__(256) void k_colsum_final(const double *part, int cols, float *out) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= cols) return;
  double acc = 0.0;
  for (int q = 0; q < CS_BLOCKS; q++) acc += part[(size_t)q * cols + c];
  out[c] = (float)acc;
}

// ---------------------------------------------------------------------------
// quasi-DEER and Jacobi sweeps: J_t replaced by its diagonal, or by zero
// ---------------------------------------------------------------------------
// The GRU Jacobian's diagonal is
//   J_ii = z_i + alpha_i W_hz[i][i] + beta_i W_hn[i][i] + gamma_i W_hr[i][i]
// (alpha, beta, gamma as in the gates kernel), so the linear recurrence
// splits into 64 scalar ones per sequence and costs O(n) per step instead of
// the chunk products' O(n^3) (Gonzalez et al. abstract: quasi-Newton
// approximations converge comparably, use less memory and are faster).
// A sweep is three launches over chunks of D64_L steps:
//  1. k_d64_gates<GM_QUASI>: W_h h_{t-1} on MFMA, the gates, the diagonal
//     J_t and r_t (stored [row][J | r]), and each chunk's aggregate per
//     channel (A = product of J, b), stored channel-major [b][i][chunk];
//  2. k_d64q_carry: one wavefront per (sequence, channel), lane = chunk: an
//     inclusive scan of the aggregates gives the state entering each chunk;
//  3. k_d64q_apply: one wavefront per chunk, lane = channel: dh_t = J_t
//     dh_{t-1} + r_t from the carry, h += dh, max |dh|.
// One wavefront per (sequence, channel); lanes take 64 chunks at a time.
__global__ __launch_bounds__(256) void k_d64q_carry(const D64Args a) {
  __shared__ int s_stop;
  if (sweep_is_stopped(a.st, &s_stop)) return;
  const int lane = threadIdx.x & 63, sc = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (sc >= a.B * 64) return;
  const int b = sc >> 6, i = sc & 63, cps = a.cps;
  const float *Ap = a.aggP + (size_t)sc * cps, *Bp = a.aggb + (size_t)sc * cps;
  float c = 0.f;  // state entering the current group of chunks
  for (int g0 = 0; g0 < cps; g0 += 64) {
    const int jj = g0 + lane;
    float A = jj < cps ? Ap[jj] : 1.f, B = jj < cps ? Bp[jj] : 0.f;
    // inclusive scan of the maps y -> A y + B, earlier lanes applied first
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float Ae = __shfl_up(A, off, 64), Be = __shfl_up(B, off, 64);
      if (lane >= off) {
        B = fmaf(A, Be, B);
        A *= Ae;
      }
    }
    const float Ai = __shfl_up(A, 1, 64), Bi = __shfl_up(B, 1, 64);
    if (jj < cps) a.carry[((size_t)b * cps + jj) * 64 + i] = lane == 0 ? c : fmaf(Ai, c, Bi);
    // lanes past the last chunk hold the identity, so lane 63 has the group's map
    c = fmaf(__shfl(A, 63, 64), c, __shfl(B, 63, 64));
  }
}

// One wavefront per chunk, lane = channel.
__global__ __launch_bounds__(256) void k_d64q_apply(const D64Args a) {
  __shared__ int s_stop;
  __shared__ unsigned s_dmax[4];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  if (sweep_is_stopped(a.st, &s_stop)) return;
  const int chunk = blockIdx.x * 4 + wid;
  unsigned dmax = 0;
  if (chunk < a.nchunks) {
    const int T = a.T, b = chunk / a.cps, j = chunk % a.cps;
    const int t0 = j * D64_L, nr = min(D64_L, T - t0);
    const size_t row0 = (size_t)b * T + t0;
    const int i = lane;
    const bool first = a.k == 1;
    float y = a.carry[(size_t)chunk * 64 + i];
    constexpr int U = 16;  // rows whose loads are issued together
    for (int s0 = 0; s0 < nr; s0 += U) {
      float Jv[U], rv[U], hv[U];
#pragma unroll
      for (int q = 0; q < U; q++) {
        const size_t row = row0 + s0 + q;
        const bool ok = s0 + q < nr;
        Jv[q] = ok ? a.gates[row * 128 + i] : 0.f;
        rv[q] = ok ? a.gates[row * 128 + 64 + i] : 0.f;
        hv[q] = (ok && !first) ? a.h[row * 64 + i] : 0.f;
      }
#pragma unroll
      for (int q = 0; q < U; q++) {
        if (s0 + q < nr) {
          y = fmaf(Jv[q], y, rv[q]);
          a.h[(row0 + s0 + q) * 64 + i] = hv[q] + y;
          const unsigned u = __float_as_uint(fabsf(y));
          dmax = u > dmax ? u : dmax;
        }
      }
    }
  }
  dmax = wave_max_u32(dmax);
  if (lane == 0) s_dmax[wid] = dmax;
  __syncthreads();
  if (tid == 0) {
    unsigned m = s_dmax[0];
    for (int q = 1; q < 4; q++) m = s_dmax[q] > m ? s_dmax[q] : m;
    max_agent(&a.st->dslot[a.k & 3][blockIdx.x % PR_DSHARDS], m);
  }
}

// ---------------------------------------------------------------------------
hipError_t launch_d64_sweep_part(D64Args &a, int part, hipStream_t s) {
  a.adjoint = 0;
  const int rows = a.B * a.T;
  if (a.approx != APX_NEWTON) {
    if (part == 0) {
      const int grid = persistent_grid<k_d64_gates<GM_QUASI>>(a.nchunks);
      if (grid <= 0) return hipErrorInvalidConfiguration;
      hipLaunchKernelGGL(k_d64_gates<GM_QUASI>, dim3(grid), dim3(256), 0, s, a);
    }
    if (part == 1) hipLaunchKernelGGL(k_d64q_carry, dim3((a.B * 64 + 3) / 4), dim3(256), 0, s, a);
    if (part == 2) hipLaunchKernelGGL(k_d64q_apply, dim3((a.nchunks + 3) / 4), dim3(256), 0, s, a);
    return hipGetLastError();
  }
  if (part == 0) {
    const int grid = persistent_grid<k_d64_gates<GM_SWEEP>>(a.nchunks);
    if (grid <= 0) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(k_d64_gates<GM_SWEEP>, dim3(grid), dim3(256), 0, s, a);
  }
  if (part == 1) hipLaunchKernelGGL(k_d64_scanA<false>, dim3((a.nchunks + 3) / 4), dim3(256), 0, s, a);
  if (part == 2) {
    hipLaunchKernelGGL(k_d64_scanB, dim3(a.B), dim3(256), 0, s, a);
    hipLaunchKernelGGL(k_d64_scanC<false>, dim3((a.nchunks + 3) / 4), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_d64_adjoint_scan(D64Args &a, hipStream_t s) {
  a.adjoint = 1;
  const int rows = a.B * a.T;
  {
    const int grid = persistent_grid<k_d64_gates<GM_ADJ>>(a.nchunks);
    if (grid <= 0) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(k_d64_gates<GM_ADJ>, dim3(grid), dim3(256), 0, s, a);
  }
  hipLaunchKernelGGL(k_d64_scanA<true>, dim3((a.nchunks + 3) / 4), dim3(256), 0, s, a);
  hipLaunchKernelGGL(k_d64_scanB, dim3(a.B), dim3(256), 0, s, a);
  hipLaunchKernelGGL(k_d64_scanC<true>, dim3((a.nchunks + 3) / 4), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_d64_adjoint_epilogue(const D64AdjArgs &a, hipStream_t s) {
  const size_t tot = (size_t)a.B * a.T * 64;
  hipLaunchKernelGGL(k_d64_adj_epi, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, s, a);
  if (a.dh0) hipLaunchKernelGGL(k_d64_dh0, dim3(a.B), dim3(64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_colsum(const float *X, int rows, int cols, float *out, double *part, hipStream_t s) {
  hipLaunchKernelGGL(k_colsum_part, dim3(CS_BLOCKS), dim3(256), 0, s, X, rows, cols, part);
  hipLaunchKernelGGL(k_colsum_final, dim3((cols + 255) / 256), dim3(256), 0, s, part, cols, out);
  return hipGetLastError();
}

}  // namespace pr

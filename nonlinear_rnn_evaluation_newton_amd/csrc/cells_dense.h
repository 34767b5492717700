// Dense-state cells for small n (state padded to N <= 8 registers): tanh RNN,
// GRU and the linear cell, with their Jacobians and vector-Jacobian products.
// Weights are read from LDS, padded with zeros so padded state entries stay 0.
//
// Cell equations follow PyTorch's RNN and GRU (the standard interface the
// Para-Seq README keeps): GRU gate order r|z|n, b_hn inside r*(.), and
// h' = (1 - z) c + z h.  The Jacobian is the one Newton linearises with
// ("Parallelizing non-linear sequential models over the sequence length",
// Approach: Jacobians give the linear operator).
#pragma once

#include "common.h"

namespace pr {

// Wh: LDS [G][N][N] row-major, bh: [G][N].  U: [G*N] (input projection incl. b_x).
template <int N, int CELL>
__device__ inline void dense_cell(const float *s, const float *U, const float *Wh, const float *bh, float *f,
                                  float *J) {
  if constexpr (CELL == C_TANH || CELL == C_LINEAR) {
#pragma unroll
    for (int i = 0; i < N; i++) {
      float a = U[i] + bh[i];
#pragma unroll
      for (int k = 0; k < N; k++) a = fmaf(Wh[i * N + k], s[k], a);
      float fi = CELL == C_TANH ? ftanh(a) : a;
      f[i] = fi;
      float da = CELL == C_TANH ? 1.f - fi * fi : 1.f;
#pragma unroll
      for (int k = 0; k < N; k++) J[i * N + k] = da * Wh[i * N + k];
    }
  } else {  // GRU
#pragma unroll
    for (int i = 0; i < N; i++) {
      float ar = U[i] + bh[i], az = U[N + i] + bh[N + i], q = bh[2 * N + i];
#pragma unroll
      for (int k = 0; k < N; k++) {
        ar = fmaf(Wh[i * N + k], s[k], ar);
        az = fmaf(Wh[(N + i) * N + k], s[k], az);
        q = fmaf(Wh[(2 * N + i) * N + k], s[k], q);
      }
      float r = fsigm(ar), z = fsigm(az);
      float c = ftanh(fmaf(r, q, U[2 * N + i]));
      f[i] = fmaf(z, s[i] - c, c);
      float al = (s[i] - c) * z * (1.f - z);
      float be = (1.f - z) * (1.f - c * c);
      float ga = be * q * r * (1.f - r);
      float bn = be * r;
#pragma unroll
      for (int k = 0; k < N; k++) {
        float v = al * Wh[(N + i) * N + k];
        v = fmaf(bn, Wh[(2 * N + i) * N + k], v);
        v = fmaf(ga, Wh[i * N + k], v);
        J[i * N + k] = (k == i) ? v + z : v;
      }
    }
  }
}

// Reverse-mode step: given lam = dL/df at (s, U), return ds = J^T lam and
// dU = dL/dU, and add dL/dW_h, dL/db_h into the accumulators.
template <int N, int CELL>
__device__ inline void dense_cell_vjp(const float *s, const float *U, const float *lam, const float *Wh,
                                      const float *bh, float *ds, float *dU, float *aWh, float *abh) {
#pragma unroll
  for (int k = 0; k < N; k++) ds[k] = 0.f;
  if constexpr (CELL == C_TANH || CELL == C_LINEAR) {
#pragma unroll
    for (int i = 0; i < N; i++) {
      float da = lam[i];
      if (CELL == C_TANH) {
        float a = U[i] + bh[i];
#pragma unroll
        for (int k = 0; k < N; k++) a = fmaf(Wh[i * N + k], s[k], a);
        float fi = ftanh(a);
        da *= 1.f - fi * fi;
      }
      dU[i] = da;
      abh[i] += da;
#pragma unroll
      for (int k = 0; k < N; k++) {
        aWh[i * N + k] = fmaf(da, s[k], aWh[i * N + k]);
        ds[k] = fmaf(da, Wh[i * N + k], ds[k]);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < N; i++) {
      float ar = U[i] + bh[i], az = U[N + i] + bh[N + i], q = bh[2 * N + i];
#pragma unroll
      for (int k = 0; k < N; k++) {
        ar = fmaf(Wh[i * N + k], s[k], ar);
        az = fmaf(Wh[(N + i) * N + k], s[k], az);
        q = fmaf(Wh[(2 * N + i) * N + k], s[k], q);
      }
      float r = fsigm(ar), z = fsigm(az);
      float c = ftanh(fmaf(r, q, U[2 * N + i]));
      float l = lam[i];
      float dz = l * (s[i] - c);
      float daz = dz * z * (1.f - z);
      float dan = l * (1.f - z) * (1.f - c * c);
      float dq = dan * r;
      float dar = dan * q * r * (1.f - r);
      ds[i] = fmaf(l, z, ds[i]);
      dU[i] = dar;
      dU[N + i] = daz;
      dU[2 * N + i] = dan;
      abh[i] += dar;
      abh[N + i] += daz;
      abh[2 * N + i] += dq;
#pragma unroll
      for (int k = 0; k < N; k++) {
        aWh[i * N + k] = fmaf(dar, s[k], aWh[i * N + k]);
        aWh[(N + i) * N + k] = fmaf(daz, s[k], aWh[(N + i) * N + k]);
        aWh[(2 * N + i) * N + k] = fmaf(dq, s[k], aWh[(2 * N + i) * N + k]);
        float v = dar * Wh[i * N + k];
        v = fmaf(daz, Wh[(N + i) * N + k], v);
        v = fmaf(dq, Wh[(2 * N + i) * N + k], v);
        ds[k] += v;
      }
    }
  }
}

}  // namespace pr

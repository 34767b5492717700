// Per-channel cells whose Jacobian is diagonal (ParaGRU) or 2x2 block-diagonal
// (CIFG/peephole ParaLSTM), as the Para-Seq README's feature table lists them.
// Channels are independent given the input projection U = W_x x + b_x, so a
// thread evaluates one channel at a time.
//
// GRU, diagonal recurrence (PyTorch gate order r|z|n, b_hn inside r*(.)):
//   r = sigm(U_r + a_r h + b_r), z = sigm(U_z + a_z h + b_z), q = a_n h + b_n,
//   c = tanh(U_n + r q), f = (1 - z) c + z h,
//   J = z + (h - c) z(1-z) a_z + (1-z)(1-c^2)(r a_n + q r(1-r) a_r).
// LSTM, coupled input/forget gate with peepholes, state (c, h):
//   f = sigm(U_f + w_f h + p_f c + b_f), g = tanh(U_g + w_g h + b_g),
//   c' = f c + (1-f) g, o = sigm(U_o + w_o h + p_o c' + b_o), h' = o tanh(c'),
//   J rows (c', h'), columns (c, h).
#pragma once

#include "common.h"

namespace pr {

struct ChanW {  // per-channel weights (fp32)
  float a0, a1, a2;  // GRU: a_r, a_z, a_n   LSTM: w_f, w_g, w_o
  float b0, b1, b2;  // recurrent biases of the three gates (only the GRU's b2 = b_hn is read: the others are in U)
  float p0, p1;      // LSTM peepholes p_f, p_o
  // the same scaled like U (see below), for the pre-activations:
  // LSTM: s0 = -L a0, s1 = 2L a1, s2 = -L a2, sp0 = -L p0, sp1 = -L p1;
  // GRU:  s0 = -L a0, s1 = -L a1, s2 = 2L a2, sb2 = 2L b2, and a0h = a0 / (2L)
  float s0, s1, s2, sp0, sp1, sb2, a0h;
};

constexpr float CH_L = 1.4426950408889634f;  // log2(e)
// Scale of gate g's pre-activation in U: -log2(e) before a sigmoid (exp2 of
// the scaled value is exp(-a)), 2 log2(e) before a tanh (or, for the GRU's
// third gate, its share of the tanh argument r q + U_n).
__host__ __device__ constexpr float chan_gate_scale(int cell_code_, int g) {
  return (cell_code_ == C_LSTM ? g == 1 : g == 2) ? 2.f * CH_L : -CH_L;
}
template <int CELL>
__device__ inline void chan_w_scale(ChanW &w) {
  constexpr int C = cell_code(CELL);
  w.s0 = chan_gate_scale(C, 0) * w.a0;
  w.s1 = chan_gate_scale(C, 1) * w.a1;
  w.s2 = chan_gate_scale(C, 2) * w.a2;
  w.sp0 = chan_gate_scale(C, 0) * w.p0;
  w.sp1 = chan_gate_scale(C, 2) * w.p1;
  w.sb2 = chan_gate_scale(C, 2) * w.b2;
  w.a0h = w.a0 * (0.5f / CH_L);
}

// U holds the input projection W_x x + b_x plus the recurrent biases of the
// gates whose pre-activation is a plain sum (the LSTM's f, g and o, the GRU's
// r and z), folded in once per solve; the GRU's b_hn stays inside r * (.).
// Each gate's column is stored scaled by chan_gate_scale, so a pre-activation
// goes to the hardware exp2 with no multiply: sigm(a) = 1 / (1 + exp2(-L a)),
// tanh(a) = 1 - 2 / (1 + exp2(2L a)).  The Jacobians use the unscaled weights.
//
// f and J at state s (SW values) with projection U (3 gates).  CELL carries
// the approximation in its upper bits (cell_apx): the LSTM's diagonal keeps
// dc'/dc and dh'/dh; zero drops every entry.
template <int CELL>
__device__ inline void chan_cell(const float *s, const float *U, const ChanW &w, float *f, float *J) {
  if constexpr (cell_code(CELL) == C_GRU_DIAG) {
    const float h = s[0];
    const float r = frcp(1.f + __builtin_amdgcn_exp2f(fmaf(w.s0, h, U[0])));
    const float z = frcp(1.f + __builtin_amdgcn_exp2f(fmaf(w.s1, h, U[1])));
    const float q2 = fmaf(w.s2, h, w.sb2);  // 2L q
    const float c = fmaf(-2.f, frcp(1.f + __builtin_amdgcn_exp2f(fmaf(r, q2, U[2]))), 1.f);
    f[0] = fmaf(z, h - c, c);
    const float be = (1.f - z) * (1.f - c * c);
    J[0] = z + (h - c) * z * (1.f - z) * w.a1 + be * r * (w.a2 + q2 * (1.f - r) * w.a0h);
  } else {  // C_LSTM
    const float c = s[0], h = s[1];
    const float fg = frcp(1.f + __builtin_amdgcn_exp2f(fmaf(w.s0, h, fmaf(w.sp0, c, U[0]))));
    const float g = fmaf(-2.f, frcp(1.f + __builtin_amdgcn_exp2f(fmaf(w.s1, h, U[1]))), 1.f);
    const float cn = fmaf(fg, c - g, g);
    const float o = frcp(1.f + __builtin_amdgcn_exp2f(fmaf(w.s2, h, fmaf(w.sp1, cn, U[2]))));
    const float tc = ftanh(cn);
    f[0] = cn;
    f[1] = o * tc;
    const float dfg = fg * (1.f - fg);
    const float dcc = fmaf((c - g) * dfg, w.p0, fg);
    const float dch = (c - g) * dfg * w.a0 + (1.f - fg) * (1.f - g * g) * w.a1;
    const float oo = o * (1.f - o) * tc;
    const float dhdcn = fmaf(oo, w.p1, o * (1.f - tc * tc));
    J[0] = dcc;
    J[1] = dch;
    J[2] = dhdcn * dcc;
    J[3] = fmaf(oo, w.a2, dhdcn * dch);
  }
  constexpr int SW = cell_code(CELL) == C_LSTM ? 2 : 1;
  if constexpr (cell_apx(CELL) == APX_ZERO) {
#pragma unroll
    for (int i = 0; i < SW * SW; i++) J[i] = 0.f;
  } else if constexpr (cell_apx(CELL) == APX_DIAG && SW == 2) {
    J[1] = 0.f;
    J[2] = 0.f;
  }
}

// Reverse-mode step: lam = dL/df; returns ds = J^T lam, dU (3 gates) and
// adds the per-channel weight gradients into acc[8] (a0 a1 a2 b0 b1 b2 p0 p1).
template <int CELL>
__device__ inline void chan_cell_vjp(const float *s, const float *U, const float *lam, const ChanW &w, float *ds,
                                     float *dU, float *acc) {
  if constexpr (CELL == C_GRU_DIAG) {
    const float h = s[0];
    const float r = frcp(1.f + __builtin_amdgcn_exp2f(fmaf(w.s0, h, U[0])));
    const float z = frcp(1.f + __builtin_amdgcn_exp2f(fmaf(w.s1, h, U[1])));
    const float q2 = fmaf(w.s2, h, w.sb2);  // 2L q
    const float q = q2 * (0.5f / CH_L);
    const float c = fmaf(-2.f, frcp(1.f + __builtin_amdgcn_exp2f(fmaf(r, q2, U[2]))), 1.f);
    const float l = lam[0];
    const float daz = l * (h - c) * z * (1.f - z);
    const float dan = l * (1.f - z) * (1.f - c * c);
    const float dq = dan * r;
    const float dar = dan * q * r * (1.f - r);
    ds[0] = l * z + dar * w.a0 + daz * w.a1 + dq * w.a2;
    dU[0] = dar;
    dU[1] = daz;
    dU[2] = dan;
    acc[0] = fmaf(dar, h, acc[0]);
    acc[1] = fmaf(daz, h, acc[1]);
    acc[2] = fmaf(dq, h, acc[2]);
    acc[3] += dar;
    acc[4] += daz;
    acc[5] += dq;
  } else {
    const float c = s[0], h = s[1];
    const float fg = frcp(1.f + __builtin_amdgcn_exp2f(fmaf(w.s0, h, fmaf(w.sp0, c, U[0]))));
    const float g = fmaf(-2.f, frcp(1.f + __builtin_amdgcn_exp2f(fmaf(w.s1, h, U[1]))), 1.f);
    const float cn = fmaf(fg, c - g, g);
    const float o = frcp(1.f + __builtin_amdgcn_exp2f(fmaf(w.s2, h, fmaf(w.sp1, cn, U[2]))));
    const float tc = ftanh(cn);
    const float lc = lam[0], lh = lam[1];
    const float dao = lh * tc * o * (1.f - o);
    const float dcn = lc + lh * o * (1.f - tc * tc) + dao * w.p1;
    const float daf = dcn * (c - g) * fg * (1.f - fg);
    const float dag = dcn * (1.f - fg) * (1.f - g * g);
    ds[0] = dcn * fg + daf * w.p0;
    ds[1] = daf * w.a0 + dag * w.a1 + dao * w.a2;
    dU[0] = daf;
    dU[1] = dag;
    dU[2] = dao;
    acc[0] = fmaf(daf, h, acc[0]);
    acc[1] = fmaf(dag, h, acc[1]);
    acc[2] = fmaf(dao, h, acc[2]);
    acc[3] += daf;
    acc[4] += dag;
    acc[5] += dao;
    acc[6] = fmaf(daf, c, acc[6]);
    acc[7] = fmaf(dao, cn, acc[7]);
  }
}

}  // namespace pr
